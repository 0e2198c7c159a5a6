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
//   gs_gram    W = P^T P per block of rows, v_mfma_f64_16x16x4 (products of fp32 values are
//              exact in fp64); partial sums are added later in a fixed order (deterministic).
//   gs_factor  modified Gram-Schmidt carried out on coefficient vectors. Column j of the
//              result is P t_j. The inner products <q_i, v_j> and the norms ||v_j|| are read
//              from the running Gram matrix, which is updated as columns are projected out.
//              This gives the upper-triangular T with P T orthonormal, T = R^-1 of the thin
//              QR. fp64, one workgroup per matrix, W and T resident in LDS, in 16-column
//              panels (one wave per diagonal panel, its pivots read through the scalar
//              unit and its column values moved by DPP row broadcasts; fp64 MFMA block
//              updates).
//              A column whose remaining squared norm is at most 2^-40 of its original squared
//              norm (or zero, or not finite) is dependent: its column of T is set to zero.
//   second pass The Gram form loses orthogonality as eps_64 times the squared condition
//              number of M q. gs_factor records whether some kept column retained less than
//              2^-20 of its squared norm; for such a matrix gs_apply stores the first result
//              in p2 instead of the outputs, and gram/factor/apply run again on p2 (the product
//              of the two triangular factors is again the thin-QR factor, so the result is the
//              same P). Matrices that need no second pass leave those launches at once.
//   gs_apply   P_hat = P T with fp64 MFMA accumulation, then the stores the products need:
//              P_hat in fp32 (caller's p), P_hat^T split bf16 hi/lo for K2, and each row's
//              power-of-two exponent for the decompression's fp16 split.
//
// Ranks above 128 (r x r no longer fits in LDS) run the same blocked recurrence on 128-column
// blocks, with W and T in global memory: the Gram matrix is formed block pair by block pair
// and summed (gs_reduce); then, per block k, gs_fdiag factors the diagonal block in LDS with
// the panel routine and gs_bgemm applies the block products of that step as fp64 MFMA GEMMs
// spread over many workgroups. gs_apply forms P_hat by 128-column blocks, and split3 finds the
// row exponents of the decompression from the fp32 factors.
#include "psgd_internal.h"

namespace psgd {
namespace {

constexpr int GS_THREADS = 256;

// ------------------------------------------------------------------------------------------
// Gram partials
// ------------------------------------------------------------------------------------------
// One work item: rows [a, a + gram_rows) of one matrix, partial index b: the upper-triangular
// 16x16 tile pairs (ti <= tj) of the rpad x rpad Gram partial, spread over the 4 waves (pair p
// to wave p % 4). Each wave runs its own statically unrolled copy of the row loop: with one
// shared loop and a per-pair "is it mine" test the compiler merged the accumulators across
// the tests (rank 80 compiled to 204 VGPRs of register moves and ran 0.45 ms against 0.21 ms
// at rank 112).
constexpr int GRAM_NW = GS_THREADS / kWave;

template <int RT, int W>
__device__ __forceinline__ void gram_rows(const GLOBAL float* __restrict__ P, GLOBAL double* __restrict__ out,
                                          int m, int rpad, int row0, int rows, int c, int g)
{
  constexpr int NP = RT * (RT + 1) / 2;
  constexpr int MINE = (NP - W + GRAM_NW - 1) / GRAM_NW;    // pairs W, W + 4, ...
  if constexpr (MINE > 0) {
    f64x4 acc[MINE];
#pragma unroll
    for (int j = 0; j < MINE; ++j) acc[j] = f64x4{0, 0, 0, 0};
    constexpr int KB = 4;                    // k steps (of 4 rows) whose loads are batched
    for (int ks = 0; ks < rows / 4; ks += KB) {
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
            if (p % GRAM_NW == W) acc[p / GRAM_NW] = mfma_f64((double)v[b][ti], (double)v[b][tj], acc[p / GRAM_NW]);
      }
    }
    // C layout of v_mfma_f64_16x16x4f64: lane 16g + c, register i holds C[g + 4i][c].
    int p = 0;
#pragma unroll
    for (int ti = 0; ti < RT; ++ti)
#pragma unroll
      for (int tj = ti; tj < RT; ++tj, ++p)
        if (p % GRAM_NW == W) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            out[(int64_t)(ti * 16 + g + 4 * i) * rpad + tj * 16 + c] = acc[p / GRAM_NW][i];
        }
  }
}

// The occupancy hint (four workgroups per CU) keeps the accumulators in ordinary VGPRs: without
// it the compiler placed them in accumulation registers, 140 registers in all at rank 112 (three
// workgroups per CU), and the kernel ran 0.226 -> 0.206 ms with it.
template <int RT>
__global__ __launch_bounds__(GS_THREADS, 4)
void k_gs_gram(const DevMat* __restrict__ mats, const Work* __restrict__ work, int pass)
{
  const Work wi = work[xcd_remap(blockIdx.x, gridDim.x)];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  if (pass && *d.reorth == 0) return;
  const GLOBAL float* __restrict__ P = gbl(pass ? d.p2 : d.p_raw);
  GLOBAL double* __restrict__ out = gbl(d.gram) + (int64_t)wi.b * d.rpad * d.rpad;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane & 15, g = lane >> 4;
  static_assert(GRAM_NW == 4, "four waves");
  switch (__builtin_amdgcn_readfirstlane(threadIdx.x / kWave)) {
    case 0: gram_rows<RT, 0>(P, out, d.m, d.rpad, wi.a, d.gram_rows, c, g); break;
    case 1: gram_rows<RT, 1>(P, out, d.m, d.rpad, wi.a, d.gram_rows, c, g); break;
    case 2: gram_rows<RT, 2>(P, out, d.m, d.rpad, wi.a, d.gram_rows, c, g); break;
    default: gram_rows<RT, 3>(P, out, d.m, d.rpad, wi.a, d.gram_rows, c, g); break;
  }
}

// W = sum of the Gram partials in part order (large ranks); also U = I (tmat) and the
// diagonal of W saved in wdiag for the factorisation's dependence test. One work item: 4096
// consecutive elements of the rpad x rpad matrix starting at a * 4096. Only the 128-column
// blocks on and above the diagonal are formed: the partials hold nothing below it, and the
// factorisation and the product P T read W and T there only.
__global__ __launch_bounds__(256)
void k_gs_reduce(const DevMat* __restrict__ mats, const Work* __restrict__ work, int pass)
{
  const Work wi = work[blockIdx.x];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  if (pass && *d.reorth == 0) return;
  const int rp = d.rpad;
  const int64_t tot = (int64_t)rp * rp;
  const int parts = d.gram_parts;
  const GLOBAL double* __restrict__ gram = gbl(d.gram);
  GLOBAL double* __restrict__ wsum = gbl(d.wsum);
  GLOBAL double* __restrict__ tmat = gbl(d.tmat);
  GLOBAL double* __restrict__ wdiag = gbl(d.wdiag);
  for (int64_t e = (int64_t)wi.a * 4096 + threadIdx.x; e < tot && e < (int64_t)(wi.a + 1) * 4096; e += 256) {
    if ((e % rp) / kBlk < (e / rp) / kBlk) continue;   // below the block diagonal
    double sum = 0.0;
#pragma unroll 8
    for (int pt = 0; pt < parts; ++pt) sum += gram[(int64_t)pt * tot + e];
    wsum[e] = sum;
    const bool diag = e / rp == e % rp;
    tmat[e] = diag ? 1.0 : 0.0;
    if (diag) wdiag[e / rp] = sum;
  }
}

// ------------------------------------------------------------------------------------------
// Gram-Schmidt on the Gram matrix (Cholesky form, T = R^-1)
// ------------------------------------------------------------------------------------------
constexpr int GSF_THREADS = 1024;

// The column recurrence: for column j, with W the Gram matrix of the residual columns, v_j is
// kept when W_jj > 2^-40 x (its squared norm before any projection) and is normalised by
// 1 / sqrt(W_jj); the later columns lose their component along it, in W and in the
// coefficient matrix T (P T has orthonormal columns; a dropped column's T column is zero).
// It runs in 16-column panels. W is held as full 16 x 16 blocks of its upper block triangle,
// beside the coefficient matrix U (initially I; block column p of U becomes block column p of
// T). For each panel p:
//   (A) one wave takes the diagonal block W_pp into registers and runs the column recurrence on
//       it with lane shuffles (no barriers), giving the panel's local factor L (T_pp = L);
//   (B) T_ip = U_ip L for i <= p, and the panel row of R, R_pj = L^T W_pj for j > p;
//   (C) U_ij -= T_ip R_pj (i <= p < j) and W_ij -= R_pi^T R_pj (p < i <= j).
// (B) and (C) are 16 x 16 x 16 block products on v_mfma_f64_16x16x4f64, one block per wave.
// In (C) wave 0 updates only W_{p+1,p+1} and then runs (A) of panel p + 1 on it, while the other
// waves update the remaining blocks (look-ahead).
// This is the right-looking blocked form of the column recurrence: every column still sees
// the residual Gram entries of its own step, so dependent columns are dropped by the same test.
constexpr int FB = 16;                 // panel width
constexpr int FBP = FB + 1;            // LDS block row pitch (doubles): column reads spread over banks
constexpr int FBS = FB * FBP;          // doubles per stored block
constexpr int FNB = kBlk / FB;         // panels at most (8)
constexpr int FNBLK = FNB * (FNB + 1) / 2;

__device__ __forceinline__ int fblk(int i, int j, int nb) {   // upper block (i <= j), packed
  return i * nb - (i * (i - 1)) / 2 + (j - i);
}

// C (+)= op(A) B for 16 x 16 blocks in LDS (pitch FBP). transA: op(A) = A^T. sub: C -= product,
// else C = product. One wave; lane 16g + c.
__device__ __forceinline__ void fblock_mm(double* C, const double* A, bool transA, const double* B,
                                          bool sub, int c, int g)
{
  f64x4 acc = {0, 0, 0, 0};
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int k = 4 * st + g;
    const double a = transA ? A[k * FBP + c] : A[c * FBP + k];
    acc = mfma_f64(a, B[k * FBP + c], acc);
  }
  // C layout of v_mfma_f64_16x16x4f64: lane 16g + c, register i holds C[g + 4i][c].
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    double& cv = C[(g + 4 * i) * FBP + c];
    cv = sub ? cv - acc[i] : acc[i];
  }
}

// Value of x in lane `lane` (wave-uniform lane index), through the scalar unit.
__device__ __forceinline__ double readlane_f64(double x, int lane) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Value of x in lane l (0..15) of the calling lane's 16-lane row (DPP row_newbcast; l must
// fold to a constant).
__device__ __forceinline__ int row_bcast_i32(int v, int l) {
  switch (l) {
#define RB(L) case L: return __builtin_amdgcn_update_dpp(0, v, 0x150 + L, 0xF, 0xF, false);
    RB(0) RB(1) RB(2) RB(3) RB(4) RB(5) RB(6) RB(7)
    RB(8) RB(9) RB(10) RB(11) RB(12) RB(13) RB(14) RB(15)
#undef RB
  }
  return v;
}
__device__ __forceinline__ double row_bcast_f64(double x, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)row_bcast_i32((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)row_bcast_i32((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// 1 / sqrt(x) for a positive normal x: the hardware estimate refined by two Newton steps
// (e = 1 - x y^2, y += y e / 2), within a few ulp. The steps commute with scaling x by a power
// of 4, so scaled inputs give exactly scaled results.
__device__ __forceinline__ double rsqrt_f64(double x) {
  double y = __builtin_amdgcn_rsq(x);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const double e = __builtin_fma(-x, y * y, 1.0);
    y = __builtin_fma(0.5 * y, e, y);
  }
  return y;
}

// The panel recurrence on nb panels held in LDS: Wb (upper block triangle of the residual
// Gram matrix), Ub (I on entry; T on return), d0 (each column's squared norm before any
// projection). All GSF_THREADS threads call it; wave 0 returns whether a kept column retained
// less than 2^-20 of its squared norm (the second-pass test), the other waves false.
__device__ __forceinline__ bool factor_panels(double* Wb, double* Ub, double* Lsh, const double* d0, int nb)
{
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  constexpr int NWV = GSF_THREADS / kWave;
  const int c = lane & 15, g = lane >> 4;
  bool again = false;
  // (A) diagonal block of panel q (wave 0): lane 16g + c holds rows g + 4i, column c, of the
  // residual Gram block (a) and of the local factor (l), which goes to Lsh. The pivot and its
  // inverse square root are wave-uniform: the pivot is read through the scalar unit and the
  // scaling is branch-free.
  auto diag = [&](int q) {
    const double* Wpp = &Wb[fblk(q, q, nb) * FBS];
    double a[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = Wpp[(g + 4 * i) * FBP + c];
      l[i] = (g + 4 * i == c) ? 1.0 : 0.0;
    }
#pragma clang loop unroll(full)
    for (int jj = 0; jj < FB; ++jj) {
      const int gj = jj & 3, ij = jj >> 2;       // holder of row jj: lanes 16 gj + x, register ij
      // The lane's column passes through an empty asm statement each step, so that the
      // per-lane conditions of the step are formed where they are used: hoisted out of the
      // unrolled steps they took 96 lane masks and spilled scalar registers.
      int cs = c;
      asm volatile("" : "+v"(cs));
      const double dj = readlane_f64(a[ij], 16 * gj + jj);
      const double dz = d0[q * FB + jj];
      const bool ok = (dz > 0.0) && (dj > kDegenerate * dz) && (dj <= 1.0e300);
      const double y = rsqrt_f64(ok ? dj : 1.0);
      const double inv = ok ? y : 0.0;
      again |= ok && dj < kReorth * dz;
      // Row jj of the residual block scaled by 1 / ||v_jj|| is r[x] = a[jj][x] inv. The
      // rank-one update a[y][x] -= r[y] r[x] and the removal of column jj from the later
      // columns of L, L[y][x] -= L[y][jj] inv r[x], both take s[x] = a[jj][x] inv^2: lane
      // 16g + c needs a[jj][c] (held in row group gj: a shuffle across rows), and a[g + 4i][jj]
      // = a[jj][g + 4i] (the block is symmetric) and L[g + 4i][jj], held by lane jj of its own
      // row group (row broadcasts). Only the later columns (c > jj) are updated; the rows up
      // to jj are updated too, which leaves them near zero and unread by the later steps.
      const double s = __shfl(a[ij], 16 * gj + cs) * inv * inv;
      const double sa = cs > jj ? s : 0.0;                 // later columns only
      const double beta = cs == jj ? inv : -sa;            // L: column jj scaled, later ones reduced
      const double alpha = cs == jj ? 0.0 : 1.0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double bl = row_bcast_f64(l[i], jj), ba = row_bcast_f64(a[i], jj);
        l[i] = __builtin_fma(bl, beta, l[i] * alpha);
        a[i] = __builtin_fma(-ba, sa, a[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) Lsh[(g + 4 * i) * FBP + c] = l[i];
  };
  if (wv == 0) diag(0);
  __syncthreads();
  for (int p = 0; p < nb; ++p) {
    // (B) T_ip = U_ip L (in place, i <= p) and R_pj = L^T W_pj (in place, j > p)
    for (int t = wv; t < nb; t += NWV) {
      if (t <= p) {
        double* U = &Ub[fblk(t, p, nb) * FBS];
        fblock_mm(U, U, false, Lsh, false, c, g);
      } else {
        double* Wj = &Wb[fblk(p, t, nb) * FBS];
        fblock_mm(Wj, Lsh, true, Wj, false, c, g);
      }
    }
    __syncthreads();
    // (C) U_ij -= T_ip R_pj (i <= p < j); W_ij -= R_pi^T R_pj (p < i <= j). Look-ahead: wave 0
    // updates the next diagonal block W_{p+1,p+1} and factors it while the other waves update
    // the remaining blocks (item nu, that diagonal block, is skipped in their list).
    const int nr = nb - p - 1;                     // block columns right of the panel
    const int nu = (p + 1) * nr, nw = nr * (nr + 1) / 2;
    if (nr > 0) {
      if (wv == 0) {
        double* Rn = &Wb[fblk(p, p + 1, nb) * FBS];
        fblock_mm(&Wb[fblk(p + 1, p + 1, nb) * FBS], Rn, true, Rn, true, c, g);
        diag(p + 1);
      } else {
        for (int t0 = wv - 1; t0 < nu + nw - 1; t0 += NWV - 1) {
          const int t = t0 < nu ? t0 : t0 + 1;
          if (t < nu) {
            const int i = t / nr, j = p + 1 + t % nr;
            fblock_mm(&Ub[fblk(i, j, nb) * FBS], &Ub[fblk(i, p, nb) * FBS], false,
                      &Wb[fblk(p, j, nb) * FBS], true, c, g);
          } else {
            int u = t - nu, i = p + 1;
            while (u >= nb - i) { u -= nb - i; ++i; }
            const int j = i + u;
            fblock_mm(&Wb[fblk(i, j, nb) * FBS], &Wb[fblk(p, i, nb) * FBS], true,
                      &Wb[fblk(p, j, nb) * FBS], true, c, g);
          }
        }
      }
    }
    __syncthreads();
  }
  return again;
}

// row-major element (row, col) of the block layout (upper block triangle only)
__device__ __forceinline__ double& fel(double* B, int row, int col, int nb) {
  return B[fblk(row / FB, col / FB, nb) * FBS + (row % FB) * FBP + col % FB];
}

// Ranks up to 128: W summed from the partials straight into LDS.
__global__ __launch_bounds__(GSF_THREADS)
void k_gs_factor(const DevMat* __restrict__ mats, const Work* __restrict__ work, int pass)
{
  const Work wi = work[blockIdx.x];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  if (pass && *d.reorth == 0) return;
  const int rp = d.rpad, nb = rp / FB;
  const int parts = d.gram_parts;
  const GLOBAL double* __restrict__ gram = gbl(d.gram);
  GLOBAL double* __restrict__ tmat = gbl(d.tmat);

  __shared__ double Wb[FNBLK * FBS];
  __shared__ double Ub[FNBLK * FBS];
  __shared__ double Lsh[FBS];
  __shared__ double diag0[kBlk];

  // W = sum of the partial Gram matrices in part order (upper block triangle); U = I.
  const int nblk = nb * (nb + 1) / 2;
  for (int e = threadIdx.x; e < nblk * FB * FB; e += GSF_THREADS) {
    const int b = e / (FB * FB), rc = e - b * FB * FB, rr = rc / FB, cc = rc - rr * FB;
    int bi = 0;
    while (fblk(bi + 1, bi + 1, nb) <= b && bi + 1 < nb) ++bi;
    const int bj = bi + (b - fblk(bi, bi, nb));
    const int row = bi * FB + rr, col = bj * FB + cc;
    double sum = 0.0;
#pragma unroll 8
    for (int pt = 0; pt < parts; ++pt) sum += gram[((int64_t)pt * rp + row) * rp + col];
    Wb[b * FBS + rr * FBP + cc] = sum;
    Ub[b * FBS + rr * FBP + cc] = (bi == bj && rr == cc) ? 1.0 : 0.0;
    if (bi == bj && rr == cc) diag0[row] = sum;
  }
  __syncthreads();

  const bool again = factor_panels(Wb, Ub, Lsh, diag0, nb);
  if (pass == 0 && threadIdx.x == 0) *gbl(d.reorth) = again ? 1 : 0;

  // T (row-major rpad x rpad; zero below the block diagonal)
  for (int e = threadIdx.x; e < rp * rp; e += GSF_THREADS) {
    const int row = e / rp, col = e - row * rp;
    tmat[e] = col / FB >= row / FB ? fel(Ub, row, col, nb) : 0.0;
  }
}

// ------------------------------------------------------------------------------------------
// Ranks above 128: the same blocked recurrence on 128-column blocks, one launch per phase.
// W (wsum, rpad x rpad, summed by k_gs_reduce, which also saves its diagonal in wdiag and sets
// tmat = I) and U (tmat) live in global memory. For each block k:
//   k_gs_fdiag(k):  the diagonal block W_kk is factored in LDS by factor_panels; its local
//                   factor L is T_kk (written into tmat);
//   k_gs_bgemm(k, 0): T_ik = U_ik L (i < k) and R_kj = L^T W_kj (j > k), in place;
//   k_gs_bgemm(k, 1): U_ij -= T_ik R_kj (i <= k < j) and W_ij -= R_ki^T R_kj (k < i <= j).
// Every product is one 128 x 128 x 128 block (ragged last block) per workgroup, so the work of
// each phase spreads over many CUs.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(GSF_THREADS)
void k_gs_fdiag(const DevMat* __restrict__ mats, const Work* __restrict__ work, int pass, int kb)
{
  const Work wi = work[blockIdx.x];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  if (pass && *d.reorth == 0) return;
  const int rp = d.rpad, k0 = kb * kBlk, bs = min(kBlk, rp - k0), nb = bs / FB;
  GLOBAL double* __restrict__ W = gbl(d.wsum);
  GLOBAL double* __restrict__ Tg = gbl(d.tmat);
  const GLOBAL double* __restrict__ wd = gbl(d.wdiag);

  __shared__ double Wb[FNBLK * FBS];
  __shared__ double Ub[FNBLK * FBS];
  __shared__ double Lsh[FBS];
  __shared__ double diag0[kBlk];

  const int nblk = nb * (nb + 1) / 2;
  for (int e = threadIdx.x; e < nblk * FB * FB; e += GSF_THREADS) {
    const int b = e / (FB * FB), rc = e - b * FB * FB, rr = rc / FB, cc = rc - rr * FB;
    int bi = 0;
    while (fblk(bi + 1, bi + 1, nb) <= b && bi + 1 < nb) ++bi;
    const int bj = bi + (b - fblk(bi, bi, nb));
    const int row = bi * FB + rr, col = bj * FB + cc;
    Wb[b * FBS + rr * FBP + cc] = W[(int64_t)(k0 + row) * rp + k0 + col];
    Ub[b * FBS + rr * FBP + cc] = (bi == bj && rr == cc) ? 1.0 : 0.0;
  }
  for (int i = threadIdx.x; i < bs; i += GSF_THREADS) diag0[i] = wd[k0 + i];
  __syncthreads();

  const bool again = factor_panels(Wb, Ub, Lsh, diag0, nb);
  if (pass == 0 && threadIdx.x == 0) {
    if (kb == 0) *gbl(d.reorth) = again ? 1 : 0;
    else if (again) *gbl(d.reorth) = 1;
  }
  for (int e = threadIdx.x; e < bs * bs; e += GSF_THREADS) {
    const int row = e / bs, col = e - row * bs;
    Tg[(int64_t)(k0 + row) * rp + k0 + col] = col / FB >= row / FB ? fel(Ub, row, col, nb) : 0.0;
  }
}

// C (bi x bj) = / -= op(A) (bi x bk) B (bk x bj), row-major with leading dimension ld; C fp64,
// A and B fp64 or fp32 (T: widened exactly on load), products and sums fp64.
// 256 threads: waves 2 x 2, each a 64 x 64 quarter of C as 4 x 4 MFMA tiles; k slices of 16
// staged in LDS (op(A) as [row][k], B as [k][col]), the next slice loaded while this one is
// multiplied. Every read of A and B happens before C is written, so C may alias A or B.
constexpr int BG_THREADS = 256;
// C (bi x bj, at most TM x TM) = op(A) B (or C -= op(A) B when sub), all row-major with leading
// dimension ld: op(A) is bi x bk (A itself, or A^T read from a bk x bi block when transA), B is
// bk x bj. Four waves, each a (TM/2) x (TM/2) quarter of C on v_mfma_f64_16x16x4f64; 16-deep
// k slices staged in LDS through buffer loads (element offsets relative to the block's first
// element; masked elements read zero). T is the element type of A and B (fp32 is widened).
template <typename T, int TM>
__device__ void bgemm_block(GLOBAL double* C, rsrc_t rA, uint32_t aoff, bool transA, rsrc_t rB,
                            uint32_t boff, bool sub, int ld, int bi, int bj, int bk)
{
  constexpr int KS = 16;
  constexpr int AP = KS + 1;               // op(A) slice pitch: column reads spread over banks
  constexpr int NT = TM / 32;              // 16 x 16 tiles per wave along each side
  constexpr int EPT = TM * KS / BG_THREADS;   // slice elements per thread and operand
  __shared__ double As[TM * AP];
  __shared__ double Bs[KS * TM];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int wm = wv & 1, wn = wv >> 1;
  const int c = lane & 15, g = lane >> 4;
  uint32_t oa[EPT], ob[EPT];
  int ka[EPT], kbb[EPT];
  bool va[EPT], vb[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int u = threadIdx.x + e * BG_THREADS;
    int row, kk;
    if (transA) { kk = u / TM; row = u % TM; } else { row = u / KS; kk = u % KS; }
    oa[e] = aoff + (transA ? (uint32_t)kk * ld + row : (uint32_t)row * ld + kk);
    ka[e] = kk;
    va[e] = row < bi;
    const int bkk = u / TM, col = u % TM;
    ob[e] = boff + (uint32_t)bkk * ld + col;
    kbb[e] = bkk;
    vb[e] = col < bj;
  }
  constexpr uint32_t ES = sizeof(T);
  auto ld1 = [&](rsrc_t r, uint32_t off) -> double {
    if constexpr (ES == 8) return __builtin_bit_cast(double, bload8(r, off));
    else return (double)__builtin_bit_cast(float, bload4(r, off));
  };
  double ra[EPT], rb[EPT];
  auto load = [&](int k0) {
    const uint32_t astep = transA ? (uint32_t)k0 * ld : (uint32_t)k0, bstep = (uint32_t)k0 * ld;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      ra[e] = ld1(rA, va[e] && k0 + ka[e] < bk ? (oa[e] + astep) * ES : kOOB);
      rb[e] = ld1(rB, vb[e] && k0 + kbb[e] < bk ? (ob[e] + bstep) * ES : kOOB);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int u = threadIdx.x + e * BG_THREADS;
      int row, kk;
      if (transA) { kk = u / TM; row = u % TM; } else { row = u / KS; kk = u % KS; }
      As[row * AP + kk] = ra[e];
      Bs[u] = rb[e];                       // [k][col]
    }
  };
  f64x4 acc[NT][NT];
#pragma unroll
  for (int a = 0; a < NT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = f64x4{0, 0, 0, 0};
  load(0);
  for (int k0 = 0; k0 < bk; k0 += KS) {
    __syncthreads();
    store();
    if (k0 + KS < bk) load(k0 + KS);
    __syncthreads();
#pragma unroll
    for (int st = 0; st < KS / 4; ++st) {
      const int k = 4 * st + g;
      double av[NT], bv[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        av[t] = As[(wm * (TM / 2) + t * 16 + c) * AP + k];
        bv[t] = Bs[k * TM + wn * (TM / 2) + t * 16 + c];
      }
#pragma unroll
      for (int tm = 0; tm < NT; ++tm)
#pragma unroll
        for (int tn = 0; tn < NT; ++tn) acc[tm][tn] = mfma_f64(av[tm], bv[tn], acc[tm][tn]);
    }
  }
  // C layout of v_mfma_f64_16x16x4f64: lane 16g + c, register i holds C[g + 4i][c].
#pragma unroll
  for (int tm = 0; tm < NT; ++tm)
#pragma unroll
    for (int tn = 0; tn < NT; ++tn)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * (TM / 2) + tm * 16 + g + 4 * i, col = wn * (TM / 2) + tn * 16 + c;
        if (row < bi && col < bj) {
          GLOBAL double* cp = C + (int64_t)row * ld + col;
          *cp = sub ? *cp - acc[tm][tn][i] : acc[tm][tn][i];
        }
      }
}

// One work item: matrix `mat`, blocks (i = a, j = b); phase 0 items with j == kb form
// T_ik = U_ik L, the others R_kj = L^T W_kj; phase 1 items with i <= kb update U, the others W.
// Phase 0 products overwrite one of their own operands, so one workgroup forms the whole
// 128 x 128 block (it reads all of its operands before it writes). Phase 1 products write a
// block that neither operand touches, so four workgroups share each, one 64 x 64 quadrant
// (c = qi | qj << 1) apiece: four times the workgroups for the few blocks of a step.
// Two workgroups per CU: 243 registers instead of 272 (accumulators out of the accumulation
// registers), so a CU holds two of these 128 x 128 block products.
template <int PHASE>
__global__ __launch_bounds__(BG_THREADS, 2)
void k_gs_bgemm(const DevMat* __restrict__ mats, const Work* __restrict__ work, int pass, int kb)
{
  constexpr int phase = PHASE;
  const Work wi = work[blockIdx.x];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  if (pass && *d.reorth == 0) return;
  const int rp = d.rpad;
  GLOBAL double* __restrict__ W = gbl(d.wsum);
  GLOBAL double* __restrict__ Tg = gbl(d.tmat);
  const int ib = wi.a, jb = wi.b;
  const int k0 = kb * kBlk, i0 = ib * kBlk, j0 = jb * kBlk;
  const int bsk = min(kBlk, rp - k0), bsi = min(kBlk, rp - i0), bsj = min(kBlk, rp - j0);
  auto blk = [&](GLOBAL double* X, int r0, int c0) { return X + (int64_t)r0 * rp + c0; };
  auto at = [&](int r0, int c0) { return (uint32_t)(r0 * rp + c0); };   // element offset
  const uint32_t bytes = (uint32_t)rp * (uint32_t)rp * 8u;
  const rsrc_t rW = make_rsrc(d.wsum, bytes), rT = make_rsrc(d.tmat, bytes);
  // The four products differ only in their operands, chosen here, so that the block product
  // is inlined once (four inlined copies took 380 VGPRs and spilled 808 bytes per lane).
  GLOBAL double* C;
  rsrc_t rA = rT, rB = rW;
  uint32_t ao, bo = at(k0, j0);
  bool transA, sub = phase != 0;
  int bi = bsi, bj = bsj;
  if (phase == 0 && jb == kb) {          // T_ik = U_ik L
    C = blk(Tg, i0, k0); ao = at(i0, k0); transA = false; rB = rT; bo = at(k0, k0); bj = bsk;
  } else if (phase == 0) {               // R_kj = L^T W_kj
    C = blk(W, k0, j0); ao = at(k0, k0); transA = true; bi = bsk;
  } else if (ib <= kb) {                 // U_ij -= T_ik R_kj
    C = blk(Tg, i0, j0); ao = at(i0, k0); transA = false;
  } else {                               // W_ij -= R_ki^T R_kj
    C = blk(W, i0, j0); rA = rW; ao = at(k0, i0); transA = true;
  }
  if constexpr (PHASE == 0) {
    bgemm_block<double, kBlk>(C, rA, ao, transA, rB, bo, sub, rp, bi, bj, bsk);
  } else {
    const int qi = wi.c & 1, qj = wi.c >> 1;
    constexpr int H = kBlk / 2;
    if (qi * H >= bi || qj * H >= bj) return;
    C += (int64_t)(qi * H) * rp + qj * H;
    ao += transA ? (uint32_t)(qi * H) : (uint32_t)(qi * H) * (uint32_t)rp;
    bo += (uint32_t)(qj * H);
    bgemm_block<double, H>(C, rA, ao, transA, rB, bo, sub, rp, min(H, bi - qi * H), min(H, bj - qj * H), bsk);
  }
}

// Gram partial of large ranks through the same block product: one work item is rows
// [a, a + gram_rows) of one matrix, partial index b, and one 64 x 64 quadrant (qi, qj) of the
// block pair (bi, bj), bi <= bj, with c = bi | bj << 8 | qi << 16 | qj << 17:
// W_part(bi, bj)[qi, qj] = P_rows(:, bi half qi)^T P_rows(:, bj half qj). Quadrants instead of
// whole 128 x 128 blocks give four times the workgroups (784 block items at r = 896 filled the
// 512 workgroup slots about 1.5 times). The quadrant of a diagonal block below its diagonal is
// skipped: the factorisation reads only the upper 16 x 16 block triangle of W, the reduction
// sums it as zeros (the partials are zeroed when the plan is made and never written there).
// Four workgroups per CU (90 registers instead of 120 with accumulation registers): 0.62 ->
// 0.55 ms at r = 896.
__global__ __launch_bounds__(BG_THREADS, 4)
void k_gs_gram_big(const DevMat* __restrict__ mats, const Work* __restrict__ work, int pass)
{
  const Work wi = work[xcd_remap(blockIdx.x, gridDim.x)];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  if (pass && *d.reorth == 0) return;
  const int rp = d.rpad;
  constexpr int H = kBlk / 2;
  const int bi = wi.c & 0xff, bj = (wi.c >> 8) & 0xff, qi = (wi.c >> 16) & 1, qj = (wi.c >> 17) & 1;
  if (bi == bj && qi > qj) return;
  const int ci0 = bi * kBlk + qi * H, cj0 = bj * kBlk + qj * H;
  if (ci0 >= rp || cj0 >= rp) return;
  const rsrc_t rP = make_rsrc(pass ? d.p2 : d.p_raw, (uint32_t)d.m * (uint32_t)rp * 4u);
  GLOBAL double* __restrict__ out = gbl(d.gram) + (int64_t)wi.b * rp * rp;
  bgemm_block<float, H>(out + (int64_t)ci0 * rp + cj0, rP, (uint32_t)(wi.a * rp + ci0), true, rP,
                        (uint32_t)(wi.a * rp + cj0), false, rp, min(H, rp - ci0), min(H, rp - cj0),
                        min(d.gram_rows, d.m - wi.a));
}

// ------------------------------------------------------------------------------------------
// P_hat = P T and the operand layouts of the two products that follow
// ------------------------------------------------------------------------------------------
// 64-row work items, four workgroups per CU (r <= 128): one workgroup's load of P and writes of
// p and P_hat^T then overlap the fp64 products of the others. With 128-row items and two
// workgroups per CU the two phases ran about back to back (0.34 ms at r = 112, 0.27 with 64).
#ifndef GSA_RA_DEF
#define GSA_RA_DEF 1
#endif
#ifndef GSA_OCC
#define GSA_OCC 4
#endif
constexpr int GSA_RA = GSA_RA_DEF;                 // 16-row tiles per wave
constexpr int GSA_ROWS = GSA_RA * 16 * (GS_THREADS / kWave);   // rows per workgroup (64)

// One work item: rows [a, a + GSA_ROWS) of P_hat and, for large ranks (BIG: RT = 8, rpad > 128),
// its 128-column block b; small ranks (rpad <= 128) take all RT column tiles at once. P is read
// into LDS by column blocks of RT tiles (one block for small ranks; blocks 0..b for large ones),
// each with all its 16-byte loads in flight at once. Each wave owns output column tiles
// {t, RT - 1 - t}: within the diagonal block of T (upper triangular) tile t costs t + 1 k tiles,
// so every pair costs RT + 1; off-diagonal blocks are dense. A wave computes its pair for all
// the item's row tiles (or a share of them when there are fewer pairs than waves), so each fragment of
// T, read from L2 one k tile ahead, feeds every row tile of the wave. The k index of an MFMA
// step is permuted within a 16-k tile (k = 16 kt + 4 g + ks), so that a lane takes its 4 A
// values of a k tile from one 16-byte LDS read. Products and sums are fp64; P_hat is rounded
// to fp32 once. Large ranks leave the row exponents of the decompression to split3 (they need
// every column block).
template <int RT, bool BIG>
__global__ __launch_bounds__(GS_THREADS, BIG ? 1 : GSA_OCC)
void k_gs_apply(const DevMat* __restrict__ mats, const Work* __restrict__ work, int pass)
{
  const Work wi = work[xcd_remap(blockIdx.x, gridDim.x)];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  const bool again = *d.reorth != 0;      // a second pass follows (pass 0) / runs (pass 1)
  if (pass && !again) return;
  const int m = d.m, r = d.r, rpad = d.rpad, mpad = d.mpad;
  const GLOBAL float* __restrict__ P = gbl(pass ? d.p2 : d.p_raw);
  const GLOBAL double* __restrict__ Tm = gbl(d.tmat);
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // uniform: scalar branches
  const int c = lane & 15, g = lane >> 4;
  const int row0 = wi.a;
  const int rows = min(GSA_ROWS, m - row0);
  constexpr int RC = RT * 16;
  constexpr int LD = RC + 4;               // LDS row pitch (floats): rows stay 16-byte aligned
  constexpr int NW = GS_THREADS / kWave;
  constexpr int NRT = GSA_ROWS / 16;       // row tiles
  const int cb = BIG ? wi.b : 0;           // output column block
  const int c0 = cb * RC;
  const int ncols = BIG ? min(RC, rpad - c0) : RC;   // output columns present (whole tiles)
  const int nto = ncols / 16;

  __shared__ __attribute__((aligned(16))) float S[GSA_ROWS * LD];

  // this wave's column-tile pair and row tiles
  constexpr int NG = (RT + 1) / 2;         // column-tile pairs
  constexpr int WPG = NG >= NW ? 1 : NW / NG;   // waves per pair
  constexpr int RPW = NRT / WPG;           // row tiles per wave
  const int gi = wv % NG, rs = wv / NG;    // pair, row share
  const bool active = wv < NG * WPG;
  const int tA = gi, tB = RT - 1 - gi;     // tB == tA for the middle tile of odd RT
  const bool haveB = active && tB < nto, haveA = active && tA < nto && tA != tB;
  f64x4 acc[2][RPW];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int a = 0; a < RPW; ++a) acc[h][a] = f64x4{0, 0, 0, 0};

  constexpr int U4 = RT * 4;               // 16-byte units per row of a column block
  constexpr int NL = GSA_ROWS * U4 / GS_THREADS;
  static_assert(NL * GS_THREADS == GSA_ROWS * U4, "load units");
  for (int kb = 0; kb <= cb; ++kb) {
    const int k0 = kb * RC;
    const int nkt = BIG ? min(RT, (rpad - k0) / 16) : RT;   // k tiles present
    // (1) columns [k0, k0 + 16 nkt) of the P tile into LDS; rows past m and missing columns zero
    if (kb > 0) __syncthreads();           // the previous block's A values have been read
    {
      f32x4 v[NL];
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int u = threadIdx.x + j * GS_THREADS, rr = u / U4, q = u - rr * U4;
        const bool ok = rr < rows && (!BIG || 4 * q < 16 * nkt);
        v[j] = ok ? *gcast<f32x4>(P + (int64_t)(row0 + rr) * rpad + k0 + 4 * q) : f32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int u = threadIdx.x + j * GS_THREADS, rr = u / U4, q = u - rr * U4;
        *reinterpret_cast<f32x4*>(&S[rr * LD + 4 * q]) = v[j];
      }
    }
    __syncthreads();
    // (2) the pair's products with this block of T: triangular on the diagonal, else dense
    const bool diag = kb == cb;
    const int endB = haveB ? (diag ? tB : nkt - 1) : -1;
    const int endA = haveA ? (diag ? tA : nkt - 1) : -1;
    const int kend = endB > endA ? endB : endA;
    if (kend >= 0) {
      double nB[4], nA[4];
      auto fetch = [&](int kt) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int64_t krow = (int64_t)(k0 + 16 * kt + 4 * g + ks) * rpad + c0;
          nB[ks] = (!BIG || kt <= endB) ? Tm[krow + 16 * tB + c] : 0.0;
          nA[ks] = kt <= endA ? Tm[krow + 16 * tA + c] : 0.0;
        }
      };
      // one k tile: UA / UB (compile-time) say which of the pair's tiles take part
      auto step = [&](int kt, auto UA, auto UB) {
        double bB[4], bA[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) { bB[ks] = nB[ks]; bA[ks] = nA[ks]; }
        if (kt < kend) fetch(kt + 1);
        f32x4 av[RPW];
#pragma unroll
        for (int a = 0; a < RPW; ++a)
          av[a] = *reinterpret_cast<const f32x4*>(&S[((rs + a * WPG) * 16 + c) * LD + 16 * kt + 4 * g]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
          for (int a = 0; a < RPW; ++a) {
            if constexpr (decltype(UB)::value) acc[1][a] = mfma_f64((double)av[a][ks], bB[ks], acc[1][a]);
            if constexpr (decltype(UA)::value) acc[0][a] = mfma_f64((double)av[a][ks], bA[ks], acc[0][a]);
          }
        }
      };
      fetch(0);
      if constexpr (BIG) {
        // k tiles where both tiles of the pair take part, then those of one of them alone (the
        // longer tile of a diagonal block, or the only one present)
        const int kboth = endA < endB ? endA : endB;
        int kt = 0;
#pragma unroll 1
        for (; kt <= kboth; ++kt) step(kt, std::true_type{}, std::true_type{});
#pragma unroll 1
        for (; kt <= endB; ++kt) step(kt, std::false_type{}, std::true_type{});
#pragma unroll 1
        for (; kt <= endA; ++kt) step(kt, std::true_type{}, std::false_type{});
      } else {
        // small ranks: tile B takes part at every k tile (kend == endB); one loop body, with the
        // test for tile A at each of its products, keeps the registers within four workgroups
        // per CU (split loops spilled)
#pragma unroll 1
        for (int kt = 0; kt <= kend; ++kt) {
          double bB[4], bA[4];
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) { bB[ks] = nB[ks]; bA[ks] = nA[ks]; }
          if (kt < kend) fetch(kt + 1);
          f32x4 av[RPW];
#pragma unroll
          for (int a = 0; a < RPW; ++a)
            av[a] = *reinterpret_cast<const f32x4*>(&S[((rs + a * WPG) * 16 + c) * LD + 16 * kt + 4 * g]);
          const bool useA = kt <= endA;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int a = 0; a < RPW; ++a) {
              acc[1][a] = mfma_f64((double)av[a][ks], bB[ks], acc[1][a]);
              if (useA) acc[0][a] = mfma_f64((double)av[a][ks], bA[ks], acc[0][a]);
            }
          }
        }
      }
    }
  }
  __syncthreads();                         // every wave has read its A values
  // C layout of v_mfma_f64_16x16x4f64: lane 16g + c, register i holds C[g + 4i][c].
#pragma unroll
  for (int a = 0; a < RPW; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = (rs + a * WPG) * 16 + g + 4 * i;
      if (haveB) S[rr * LD + 16 * tB + c] = (float)acc[1][a][i];
      if (haveA) S[rr * LD + 16 * tA + c] = (float)acc[0][a][i];
    }
  __syncthreads();

  const int u4c = ncols / 4;               // 16-byte units of a row present
  if (pass == 0 && again) {
    // first pass of a matrix that needs two: the result is the second pass's input
    GLOBAL float* __restrict__ p2 = gbl(d.p2);
    for (int u = threadIdx.x; u < rows * u4c; u += GS_THREADS) {
      const int rr = u / u4c, q = u - rr * u4c;
      *gcast<f32x4>(p2 + (int64_t)(row0 + rr) * rpad + c0 + 4 * q) = *reinterpret_cast<const f32x4*>(&S[rr * LD + 4 * q]);
    }
    return;
  }

  // (a) fp32 P_hat, m x r row-major (this block's columns below r)
  GLOBAL float* __restrict__ pout = gbl(d.p);
  const int pc = max(0, min(ncols, r - c0));
  if ((r & 3) == 0) {
    const int ur = pc / 4;
    for (int u = threadIdx.x; u < rows * ur; u += GS_THREADS) {
      const int rr = u / ur, q = u - rr * ur;
      *gcast<f32x4>(pout + (int64_t)(row0 + rr) * r + c0 + 4 * q) = *reinterpret_cast<const f32x4*>(&S[rr * LD + 4 * q]);
    }
  } else {
    for (int u = threadIdx.x; u < rows * pc; u += GS_THREADS) {
      const int rr = u / pc, cc = u - rr * pc;
      pout[(int64_t)(row0 + rr) * r + c0 + cc] = S[rr * LD + cc];
    }
  }
  // (b) P_hat^T split bf16 hi/lo, rpad x mpad: 8 consecutive rows of one column per store
  GLOBAL uint16_t* __restrict__ pth = gbl(d.pt_hi);
  GLOBAL uint16_t* __restrict__ ptl = gbl(d.pt_lo);
  for (int idx = threadIdx.x; idx < ncols * (GSA_ROWS / 8); idx += GS_THREADS) {
    const int col = idx / (GSA_ROWS / 8), r8 = (idx % (GSA_ROWS / 8)) * 8;
    if (row0 + r8 >= mpad) continue;
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = S[(r8 + 2 * e) * LD + col], x1 = S[(r8 + 2 * e + 1) * LD + col];
      const __bf16 h0 = (__bf16)x0, h1 = (__bf16)x1;
      h[e] = bf16_bits(h0) | ((uint32_t)bf16_bits(h1) << 16);
      l[e] = bf16_bits((__bf16)(x0 - (float)h0)) | ((uint32_t)bf16_bits((__bf16)(x1 - (float)h1)) << 16);
    }
    *gcast<u32x4>(pth + (int64_t)(c0 + col) * mpad + row0 + r8) = u32x4{h[0], h[1], h[2], h[3]};
    *gcast<u32x4>(ptl + (int64_t)(c0 + col) * mpad + row0 + r8) = u32x4{l[0], l[1], l[2], l[3]};
  }
  if constexpr (BIG) return;
  // (c) row exponents of the decompression operand: the power of two that brings the row's
  // largest entry into [2^13, 2^14) before the decompression splits it into fp16 hi + lo
  GLOBAL int32_t* __restrict__ p3e = gbl(d.p3_exp);
  if ((int)threadIdx.x < rows) {
    float amax = 0.0f;
    for (int cc = 0; cc < RC; ++cc) amax = fmaxf(amax, fabsf(S[threadIdx.x * LD + cc]));
    p3e[row0 + threadIdx.x] = fp16_row_exponent(amax);
  }
}

// Row exponents of the decompression operands (ranks above one chunk, or q_next after the
// caller changed it): for each row of P_hat (which = 0, from p) or of Q' (which = 1, from
// q_next), the power of two that brings its largest entry into [2^13, 2^14). Ranks above one
// chunk also get the row, scaled by that power, split into fp16 hi + lo once here, for the
// decompression to copy into its stages: kpad3 ranks per row as 16-byte pairs per 8 ranks (hi,
// then lo), ranks past r zero; the same arithmetic as the decompression's own split of fp32
// factors. One work item: 64 rows [a, a + 64) of matrix `mat`, which = b; one wave per row at
// a time, each lane holding up to two 8-rank units of the row.
constexpr int S3_UNITS = kMaxRank / 8 / kWave;   // 8-rank units per lane
__global__ __launch_bounds__(256)
void k_split3(const DevMat* __restrict__ mats, const Work* __restrict__ work)
{
  const Work wi = work[blockIdx.x];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  const int r = d.r, kpad3 = d.kpad3;
  const bool isq = wi.b != 0;
  const int rows = isq ? d.n : d.m;
  const GLOBAL float* __restrict__ src = gbl(isq ? d.q_next : d.p);
  GLOBAL int32_t* __restrict__ ex = gbl(isq ? d.q3_exp : d.p3_exp);
  GLOBAL uint16_t* __restrict__ halves = gbl(isq ? d.q3h : d.p3h);   // NULL: exponents only
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const bool rvec = (r & 3) == 0;               // rows start 16-byte aligned
  for (int row = wi.a + wv; row < wi.a + 64 && row < rows; row += 4) {
    const GLOBAL float* __restrict__ x = src + (int64_t)row * r;
    float amax = 0.0f;
    f32x4 v[S3_UNITS][2];
#pragma unroll
    for (int u = 0; u < S3_UNITS; ++u) {
      const int k = 8 * (lane + kWave * u);
      if (rvec && k + 8 <= r) {
        v[u][0] = *gcast<f32x4>(x + k);
        v[u][1] = *gcast<f32x4>(x + k + 4);
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) v[u][t >> 2][t & 3] = k + t < r ? x[k + t] : 0.0f;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) amax = fmaxf(amax, fmaxf(fabsf(v[u][0][t]), fabsf(v[u][1][t])));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const int e = fp16_row_exponent(amax);
    if (lane == 0) ex[row] = e;
    if (halves != nullptr) {
      GLOBAL uint16_t* __restrict__ hrow = halves + (int64_t)row * kpad3 * 2;
#pragma unroll
      for (int u = 0; u < S3_UNITS; ++u) {
        const int k = 8 * (lane + kWave * u);
        if (k >= kpad3) continue;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          f32x4 xs;
#pragma unroll
          for (int t = 0; t < 4; ++t) xs[t] = ldexpf(v[u][h][t], e);
          const f16x4 hi = __builtin_convertvector(xs, f16x4);
          const f16x4 lo = __builtin_convertvector(xs - __builtin_convertvector(hi, f32x4), f16x4);
          *gcast<f16x4>(hrow + 2 * k + 4 * h) = hi;
          *gcast<f16x4>(hrow + 2 * k + 8 + 4 * h) = lo;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gs_gram(int rt, bool big, int pass, const DevMat* mats, const Work* work, int n_work, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  const dim3 grid(n_work), block(GS_THREADS);
  if (big) {
    k_gs_gram_big<<<grid, dim3(BG_THREADS), 0, s>>>(mats, work, pass);
    return hipGetLastError();
  }
  switch (rt) {
#define CASE(R) case R: k_gs_gram<R><<<grid, block, 0, s>>>(mats, work, pass); break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
#undef CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gs_reduce(int pass, const DevMat* mats, const Work* work, int n_work, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  k_gs_reduce<<<dim3(n_work), dim3(256), 0, s>>>(mats, work, pass);
  return hipGetLastError();
}

hipError_t launch_gs_factor(int pass, const DevMat* mats, const Work* work, int n_work, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  k_gs_factor<<<dim3(n_work), dim3(GSF_THREADS), 0, s>>>(mats, work, pass);
  return hipGetLastError();
}

hipError_t launch_gs_fdiag(int pass, int kb, const DevMat* mats, const Work* work, int n_work, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  k_gs_fdiag<<<dim3(n_work), dim3(GSF_THREADS), 0, s>>>(mats, work, pass, kb);
  return hipGetLastError();
}

hipError_t launch_gs_bgemm(int pass, int kb, int phase, const DevMat* mats, const Work* work, int n_work,
                           hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  if (phase == 0) k_gs_bgemm<0><<<dim3(n_work), dim3(BG_THREADS), 0, s>>>(mats, work, pass, kb);
  else k_gs_bgemm<1><<<dim3(n_work), dim3(BG_THREADS), 0, s>>>(mats, work, pass, kb);
  return hipGetLastError();
}

hipError_t launch_gs_apply(int rt, bool big, int pass, const DevMat* mats, const Work* work, int n_work, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  const dim3 grid(n_work), block(GS_THREADS);
  if (big) {
    k_gs_apply<kMaxRankTiles, true><<<grid, block, 0, s>>>(mats, work, pass);
    return hipGetLastError();
  }
  switch (rt) {
#define CASE(R) case R: k_gs_apply<R, false><<<grid, block, 0, s>>>(mats, work, pass); break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
#undef CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_split3(const DevMat* mats, const Work* work, int n_work, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  k_split3<<<dim3(n_work), dim3(256), 0, s>>>(mats, work);
  return hipGetLastError();
}

int gs_apply_rows_per_block() { return GSA_ROWS; }

}  // namespace psgd
