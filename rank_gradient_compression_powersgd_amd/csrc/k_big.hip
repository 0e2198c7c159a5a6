// Ranks above one 128-column chunk: the two factor products P = M q and Q' = M^T P as GEMMs
// on operands split into bfloat16 halves once per step.
//
// The products are the P·Q factorisation of the Korean summary of the DALL·E paper (section
// "Distributed Optimization"); the error-buffer accumulation M = s_b G + E and its finite
// check come from "Zero-Shot Text-to-Image Generation — 中文验证版" (section 证据).
//
// At r = 128 and below the products stream G and E once each and are bound by HBM bandwidth
// (the M q and M^T P kernels). At higher ranks those kernels walk G and E once per 128-rank
// chunk and convert M to bf16 halves in every pass; the conversions, not the bytes, then
// bound them. Here M is formed and split once:
//   k_split_m   M = s_b G + E -> M_hi, M_lo (m x n, row-major, bf16, zero-padded) and the
//               per-matrix flag "G or E holds inf/NaN";
//   k_split_qt  q (n x r fp32) -> q^T split into bf16 halves (rpad x n);
//   k_gemm_nt   C = A B^T over K with bf16 halves, three products A_hi B_hi + A_hi B_lo +
//               A_lo B_hi accumulated in fp32 (as the streaming kernels do): P_raw = M (q^T)^T
//               with both operands K-contiguous, and q_next = M^T (P^T)^T, P^T being the halves
//               the orthonormal-factor kernel writes and A = M^T read from M's row-major halves
//               (K-outer) through gfx950's transposing LDS read, so no transposed copy of M is
//               written.
#include "psgd_internal.h"

namespace psgd {
namespace {

constexpr int ST = 64;          // split tile: 64 x 64 elements
constexpr int ST_THREADS = 256;
constexpr int STP = ST + 8;     // LDS row pitch of the q transpose tile (bf16), 16-byte rows apart

// 64 x 64 tile (rows i0.., columns j0..) of the padded M range: 16 lanes per row, 4 columns
// each, 16 rows per step, 4 steps. Rows past m and columns past n read zeros (buffer
// descriptors), so the padding of M is written as zeros.
template <int GT>
__global__ __launch_bounds__(ST_THREADS)
void k_split_m(const DevMat* __restrict__ mats, const Work* __restrict__ work,
               const float* __restrict__ scale, uint8_t* __restrict__ flags)
{
  const Work wi = work[xcd_remap(blockIdx.x, gridDim.x)];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  const int m = d.m, n = d.n, i0 = wi.a, j0 = wi.b;
  const int ldg = (int)d.ld_grad, lde = (int)d.ld_err;
  const int ldm = d.npad_b;
  const rsrc_t rg = make_rsrc(d.grad, d.g_bytes);
  const rsrc_t re = make_rsrc(d.err, d.e_bytes);
  const float s = d.grad ? scale[d.block] : 0.0f;   // in-place matrices: E already holds M
  constexpr int GB = GradIO<GT>::kBytes;
  const int lu = threadIdx.x & 15, lr = threadIdx.x >> 4;
  GLOBAL uint16_t* __restrict__ mh = gbl(d.mh);
  GLOBAL uint16_t* __restrict__ ml = gbl(d.ml);
  bool bad = false;
  GradVec<GT, 4> gv[4];
  GradVec<G_F32, 4> ev[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int row = i0 + lr + 16 * st, col = j0 + 4 * lu;
    const bool ok = row < m && col < n;           // n % 8 == 0: col < n covers col + 3
    gv[st].load(rg, ok ? (uint32_t)(row * ldg + col) * GB : kOOB);
    ev[st].load(re, ok ? (uint32_t)(row * lde + col) * 4u : kOOB);
  }
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int row = i0 + lr + 16 * st, col = j0 + 4 * lu;
    const f32x4 gf = gv[st].f32(), ef = ev[st].f32();
    f32x4 mv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bad |= nonfinite(gf[e]) || nonfinite(ef[e]);
      mv[e] = __builtin_fmaf(s, gf[e], ef[e]);
    }
    const bf16x4 hi = __builtin_convertvector(mv, bf16x4);
    const bf16x4 lo = __builtin_convertvector(mv - __builtin_convertvector(hi, f32x4), bf16x4);
    *gcast<u32x2>(mh + (int64_t)row * ldm + col) = __builtin_bit_cast(u32x2, hi);
    *gcast<u32x2>(ml + (int64_t)row * ldm + col) = __builtin_bit_cast(u32x2, lo);
  }
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && (threadIdx.x & (kWave - 1)) == 0) gbl(flags)[wi.mat] = 1;
}

// 64 x 64 tile of q (rows = k of the M q product i0.., ranks j0..) -> q^T halves (rpad_b x
// npad_b, every element written). Ranks past r and rows past n read zeros.
__global__ __launch_bounds__(ST_THREADS)
void k_split_qt(const DevMat* __restrict__ mats, const Work* __restrict__ work)
{
  const Work wi = work[xcd_remap(blockIdx.x, gridDim.x)];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  const int n = d.n, r = d.r, i0 = wi.a, j0 = wi.b, ldq = d.npad_b;
  const rsrc_t rq = make_rsrc(d.q, (uint32_t)n * (uint32_t)r * 4u);
  const int lu = threadIdx.x & 15, lr = threadIdx.x >> 4;
  __shared__ __attribute__((aligned(16))) uint16_t th[ST][STP], tl[ST][STP];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int rr = lr + 16 * st, row = i0 + rr, rank = j0 + 4 * lu;
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = __builtin_bit_cast(float, bload4(rq, row < n && rank + e < r ? (uint32_t)(row * r + rank + e) * 4u : kOOB));
    const bf16x4 hi = __builtin_convertvector(v, bf16x4);
    const bf16x4 lo = __builtin_convertvector(v - __builtin_convertvector(hi, f32x4), bf16x4);
    *reinterpret_cast<bf16x4*>(&th[rr][4 * lu]) = hi;
    *reinterpret_cast<bf16x4*>(&tl[rr][4 * lu]) = lo;
  }
  __syncthreads();
  GLOBAL uint16_t* __restrict__ qh = gbl(d.qth);
  GLOBAL uint16_t* __restrict__ ql = gbl(d.qtl);
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int jj = lr + 16 * st, ii = 4 * lu;
    uint16_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) { h[e] = th[ii + e][jj]; l[e] = tl[ii + e][jj]; }
    const u32x2 hv = {(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
    const u32x2 lv = {(uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16)};
    *gcast<u32x2>(qh + (int64_t)(j0 + jj) * ldq + i0 + ii) = hv;
    *gcast<u32x2>(ql + (int64_t)(j0 + jj) * ldq + i0 + ii) = lv;
  }
}

// ---- C = A B^T on split bf16 operands -----------------------------------------------------
#ifndef GEMM_WRT
#define GEMM_WRT 4
#endif
constexpr int WRT = GEMM_WRT;                  // 16-row A tiles per wave
constexpr int GT_M = 2 * WRT * 16, GT_N = 128; // C tile; 2 x 2 waves of (16 WRT) x 64
constexpr int UA = GT_M / 64, UB = GT_N / 64;  // 16-byte staging units per thread and operand half
constexpr int GM_THREADS = 256;
constexpr int GK = 32;                         // K per stage: LDS row = 32 bf16 = 4 16-byte units
// physical 16-byte unit of logical unit q in LDS row rr (64-byte rows): the 8 lanes of one LDS
// pass read 8 consecutive rows and hit the 8 distinct 16-byte groups of the 32 banks
__device__ __forceinline__ int swzg(int rr, int q) { return q ^ ((rr >> 1) & 3); }
// K-outer A (LDS row = one k, 128 bf16 = 256 bytes = all 64 banks): physical 16-byte unit of
// logical unit q in row k. A transposing read touches 32 bytes (a pair of units) in each of
// 16 rows, k = 8 g + 4 h + t (g, t = 0..3); the pair index is XOR-ed with t + 4 (g & 1), so the
// 8 rows of lanes 0..31 (g = 0, 1), and those of lanes 32..63, land on 8 distinct pairs: all
// 64 banks once. Stores of whole rows stay conflict-free (a permutation within the row).
__device__ __forceinline__ int swzt(int k, int q) { return q ^ (2 * ((k & 3) | (((k >> 3) & 1) << 2))); }

struct GemmArgs {
  rsrc_t ah, al, bh, bl;        // operand halves: A rows x K (K x A rows when K-outer), B rows x K
  int lda, ldb, K;              // leading dimensions (elements), K a multiple of GK
  GLOBAL float* c; int ldc, crows, ccols;
};

__device__ __forceinline__ GemmArgs gemm_args(const DevMat& d, int which) {
  GemmArgs g;
  if (which == 0) {             // P_raw (m x rpad) = M q:  A = M (mpad x npad_b), B = q^T (rpad_b x npad_b)
    const uint32_t ab = (uint32_t)d.mpad * (uint32_t)d.npad_b * 2u, bb = (uint32_t)d.rpad_b * (uint32_t)d.npad_b * 2u;
    g.ah = make_rsrc(d.mh, ab); g.al = make_rsrc(d.ml, ab);
    g.bh = make_rsrc(d.qth, bb); g.bl = make_rsrc(d.qtl, bb);
    g.lda = d.npad_b; g.ldb = d.npad_b; g.K = d.npad_b;
    g.c = gbl(d.p_raw); g.ldc = d.rpad; g.crows = d.m; g.ccols = d.rpad;
  } else {                      // q_next (n x r) = M^T P:  A = M^T, K-outer (M, mpad x npad_b), B = P^T (rpad x mpad)
    const uint32_t ab = (uint32_t)d.mpad * (uint32_t)d.npad_b * 2u, bb = (uint32_t)d.rpad * (uint32_t)d.mpad * 2u;
    g.ah = make_rsrc(d.mh, ab); g.al = make_rsrc(d.ml, ab);
    g.bh = make_rsrc(d.pt_hi, bb); g.bl = make_rsrc(d.pt_lo, bb);
    g.lda = d.npad_b; g.ldb = d.mpad; g.K = d.mpad;
    g.c = gbl(d.q_next); g.ldc = d.r; g.crows = d.n; g.ccols = d.r;
  }
  return g;
}

// gfx950's transposing LDS read (ds_read_b64_tr_b16): each lane names 8 bytes (4 consecutive
// 16-bit elements of one LDS row); within every 16 lanes, lane j receives element j % 4 of the
// 8-byte pieces named by lanes j / 4, j / 4 + 4, j / 4 + 8 and j / 4 + 12, in that order. If
// lane s of the 16 names row k0 + s / 4 at column c0 + 4 (s % 4), lane j therefore receives
// rows k0 .. k0 + 3 of column c0 + j: 4 consecutive k of one row of A^T, as an MFMA operand
// takes them.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// One work item: matrix `mat`, C tile rows a.., columns b.. of the product AT selects: M q
// (AT false) or M^T P (AT true, A stored K-outer: row k of M holds A[.][k]; staged as GK LDS
// rows of GT_M elements and read with the transposing LDS read).
template <bool AT>
__global__ __launch_bounds__(GM_THREADS, WRT == 4 ? 2 : 1)
void k_gemm_nt(const DevMat* __restrict__ mats, const Work* __restrict__ work)
{
  const Work wi = work[xcd_remap(blockIdx.x, gridDim.x)];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  const GemmArgs ga = gemm_args(d, AT ? 1 : 0);
  const int i0 = wi.a, j0 = wi.b;
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int wm = wv & 1, wn = wv >> 1;
  const int c = lane & 15, g = lane >> 4;

  constexpr int ATP = GT_M;                                       // K-outer A: LDS row pitch
  constexpr int A_ELEMS = AT ? GK * ATP : GT_M * GK;              // one buffer, one half
  __shared__ __attribute__((aligned(16))) uint16_t ldsA[2][2][A_ELEMS];     // [buf][hi/lo][...]
  __shared__ __attribute__((aligned(16))) uint16_t ldsB[2][2][GT_N][GK];

  // staging: a 16-byte unit is 8 consecutive k of one row; 4 units per row, UA (UB) per
  // thread and operand half. Rows past the operand's padded extent read zeros. Two register
  // sets hold the next two stages, so a stage's loads have two stages of products to arrive.
  // K-outer A: a unit is 8 consecutive A rows at one k; 16 units per k (GT_M / 8 = 16), and
  // A rows past lda (the padded row length of the source) read zeros.
  struct Regs { u32x4 a[UA][2], b[UB][2]; };     // [unit][hi/lo]
  Regs R0, R1;
  uint32_t aoff[UA], boff[UB];
  int arow[UA], aq[UA], brow[UB], bq[UB];
  bool aok[UA];
#pragma unroll
  for (int j = 0; j < UA; ++j) {
    const int u = threadIdx.x + GM_THREADS * j;
    if constexpr (AT) {
      arow[j] = u >> 4;                           // k within the stage
      aq[j] = u & 15;                             // unit along the A rows
      aok[j] = i0 + 8 * aq[j] < ga.lda;
      aoff[j] = ((uint32_t)arow[j] * (uint32_t)ga.lda + (uint32_t)(i0 + 8 * aq[j])) * 2u;
    } else {
      arow[j] = u >> 2;
      aq[j] = u & 3;
      aok[j] = true;
      aoff[j] = ((uint32_t)(i0 + arow[j]) * (uint32_t)ga.lda + 8u * aq[j]) * 2u;
    }
  }
#pragma unroll
  for (int j = 0; j < UB; ++j) {
    const int u = threadIdx.x + GM_THREADS * j;
    brow[j] = u >> 2;
    bq[j] = u & 3;
    boff[j] = ((uint32_t)(j0 + brow[j]) * (uint32_t)ga.ldb + 8u * bq[j]) * 2u;
  }
  auto load_stage = [&](Regs& R, int k0) {
    const uint32_t kb = (uint32_t)k0 * 2u;
    const uint32_t kba = AT ? (uint32_t)k0 * (uint32_t)ga.lda * 2u : kb;
#pragma unroll
    for (int j = 0; j < UA; ++j) {
      R.a[j][0] = bload16(ga.ah, aok[j] ? aoff[j] + kba : kOOB);
      R.a[j][1] = bload16(ga.al, aok[j] ? aoff[j] + kba : kOOB);
    }
#pragma unroll
    for (int j = 0; j < UB; ++j) {
      R.b[j][0] = bload16(ga.bh, boff[j] + kb);
      R.b[j][1] = bload16(ga.bl, boff[j] + kb);
    }
  };
  auto store_stage = [&](const Regs& R, int buf) {
#pragma unroll
    for (int j = 0; j < UA; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int off = AT ? arow[j] * ATP + 8 * swzt(arow[j], aq[j]) : arow[j] * GK + 8 * swzg(arow[j], aq[j]);
        *reinterpret_cast<u32x4*>(&ldsA[buf][h][off]) = R.a[j][h];
      }
#pragma unroll
    for (int j = 0; j < UB; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *reinterpret_cast<u32x4*>(&ldsB[buf][h][brow[j]][8 * swzg(brow[j], bq[j])]) = R.b[j][h];
  };

  f32x4 acc[WRT][4];   // [A tile][B tile]
#pragma unroll
  for (int a = 0; a < WRT; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0, 0, 0, 0};
  auto compute = [&](int buf) {
    bf16x8 bh[4], bl[4];
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) {
      const int rb = wn * 64 + jn * 16 + c;
      bh[jn] = *reinterpret_cast<const bf16x8*>(&ldsB[buf][0][rb][8 * swzg(rb, g)]);
      bl[jn] = *reinterpret_cast<const bf16x8*>(&ldsB[buf][1][rb][8 * swzg(rb, g)]);
    }
#pragma unroll
    for (int im = 0; im < WRT; ++im) {
      bf16x8 ah, al;
      if constexpr (AT) {
        // rows k = 8 g .. 8 g + 7 of A row wm * 16 WRT + 16 im + c, in two transposing reads
        // (rows k and k + 4 share their swizzle)
        const int k = 8 * g + (c >> 2), q = (wm * (WRT * 16) + im * 16) / 8 + ((c & 3) >> 1);
        const int off = k * ATP + 8 * swzt(k, q) + 4 * (c & 1);
        const i16x4 h0 = lds_read_tr16(&ldsA[buf][0][off]), h1 = lds_read_tr16(&ldsA[buf][0][off + 4 * ATP]);
        const i16x4 l0 = lds_read_tr16(&ldsA[buf][1][off]), l1 = lds_read_tr16(&ldsA[buf][1][off + 4 * ATP]);
        ah = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
        al = __builtin_bit_cast(bf16x8, __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7));
      } else {
        const int ra = wm * (WRT * 16) + im * 16 + c;
        ah = *reinterpret_cast<const bf16x8*>(&ldsA[buf][0][ra * GK + 8 * swzg(ra, g)]);
        al = *reinterpret_cast<const bf16x8*>(&ldsA[buf][1][ra * GK + 8 * swzg(ra, g)]);
      }
#pragma unroll
      for (int jn = 0; jn < 4; ++jn) {
        acc[im][jn] = mfma_bf16(ah, bh[jn], acc[im][jn]);
        acc[im][jn] = mfma_bf16(ah, bl[jn], acc[im][jn]);
        acc[im][jn] = mfma_bf16(al, bh[jn], acc[im][jn]);
      }
    }
  };

  const int nsteps = ga.K / GK;
  // stage s lives in LDS buffer s & 1 and arrives in register set s & 1
  load_stage(R0, 0);
  if (nsteps > 1) load_stage(R1, GK);
  store_stage(R0, 0);
  __syncthreads();
  for (int ks = 0; ks < nsteps; ks += 2) {
    if (ks + 2 < nsteps) load_stage(R0, (ks + 2) * GK);
    compute(0);
    if (ks + 1 < nsteps) store_stage(R1, 1);
    __syncthreads();
    if (ks + 1 < nsteps) {
      if (ks + 3 < nsteps) load_stage(R1, (ks + 3) * GK);
      compute(1);
      if (ks + 2 < nsteps) store_stage(R0, 0);
      __syncthreads();
    }
  }

  // C layout of v_mfma_f32_16x16x32_bf16: lane holds rows 4g..4g+3 (of A), column c (of B).
#pragma unroll
  for (int im = 0; im < WRT; ++im)
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) {
      const int col = j0 + wn * 64 + jn * 16 + c;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = i0 + wm * (WRT * 16) + im * 16 + 4 * g + i;
        if (row < ga.crows && col < ga.ccols) ga.c[(int64_t)row * ga.ldc + col] = acc[im][jn][i];
      }
    }
}

}  // namespace

int big_split_tile() { return ST; }
int big_gemm_tile_m() { return GT_M; }
int big_gemm_tile_n() { return GT_N; }

hipError_t launch_split_m(int gt, const DevMat* mats, const Work* work, int n_work, const float* scale,
                          uint8_t* flags, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  const dim3 grid(n_work), block(ST_THREADS);
  switch (gt) {
    case G_F16: k_split_m<G_F16><<<grid, block, 0, s>>>(mats, work, scale, flags); break;
    case G_BF16: k_split_m<G_BF16><<<grid, block, 0, s>>>(mats, work, scale, flags); break;
    case G_F32: k_split_m<G_F32><<<grid, block, 0, s>>>(mats, work, scale, flags); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_split_qt(const DevMat* mats, const Work* work, int n_work, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  k_split_qt<<<dim3(n_work), dim3(ST_THREADS), 0, s>>>(mats, work);
  return hipGetLastError();
}

hipError_t launch_gemm_nt(const DevMat* mats, const Work* work, int n_work, bool a_k_outer, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  if (a_k_outer) k_gemm_nt<true><<<dim3(n_work), dim3(GM_THREADS), 0, s>>>(mats, work);
  else k_gemm_nt<false><<<dim3(n_work), dim3(GM_THREADS), 0, s>>>(mats, work);
  return hipGetLastError();
}

}  // namespace psgd
