// K3: decompression D = P Q'^T with fp32-accurate products, and the error-feedback write-back
// E = M - D with M = s_b G + E recomputed; optional D output.
//
// "Zero-Shot Text-to-Image Generation — 中文验证版" (section 证据) asks for 32-bit products in
// the decompressed gradient. Both factors were stored as fp16 hi + lo pairs of rows scaled by
// powers of two (|x - hi - lo| <= 2^-22 |x|), and three fp16 MFMA products (hi*hi + hi*lo +
// lo*hi) with fp32 accumulation reproduce fp32 products to about 2^-21. The power-of-two row
// scales are removed exactly with ldexp.
//
// The tile is computed transposed, D^T = Q' P^T, so the MFMA C layout gives every lane 4
// consecutive columns of one row of D. The finished tile is passed through LDS so that the
// G/E/out traffic runs in whole 128-byte lines: in the C layout one wave instruction would
// touch half of a line in each of 16 rows, which HBM serves at a markedly lower rate. G, E and
// out go through buffer descriptors: ragged edges read zeros and drop their stores in
// hardware, so the epilogue issues the loads of all its rows at once and has no branches.
//
// Skip: the device-side skip word is read first. A skipped step zeroes the error buffer over
// the tile and writes nothing else (the error buffer is zeroed on non-finite values: Korean
// summary of the paper, section "Distributed Optimization").
#include "psgd_internal.h"

namespace psgd {
namespace {

#ifndef K3_WM
#define K3_WM 2      // waves along m
#endif
#ifndef K3_WN
#define K3_WN 2      // waves along n; each wave computes a 64 x 64 tile
#endif
#ifndef K3_OCC
#define K3_OCC 2     // workgroups per CU the register budget is sized for
#endif
constexpr int K3_TM = K3_WM * 64, K3_TN = K3_WN * 64;
constexpr int K3_THREADS = K3_WM * K3_WN * kWave;
constexpr int LDS_K = 32;                // LDS row = 32 fp16 = 4 16-byte units, XOR-swizzled
constexpr int K3_DTP = K3_TN + 4;        // D tile row pitch (floats), rows 16-byte aligned
constexpr int kStageQBytes = 2 * 2 * K3_TN * LDS_K * 2;
constexpr int kStageBytes = kStageQBytes + 2 * 2 * K3_TM * LDS_K * 2;
constexpr int kTileBytes = K3_TM * K3_DTP * 4;
constexpr int kLdsBytes = kStageBytes > kTileBytes ? kStageBytes : kTileBytes;
// Physical unit of logical unit q in row rr: 16 lanes reading 16 consecutive rows (one unit
// each) or writing 4 rows (4 units each) hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz3(int rr, int q) { return q ^ ((rr >> 2) & 3); }

// G, E and out are streamed with the non-temporal policy: they are touched once, and evicting
// them first keeps the factor tiles, which neighbouring workgroups re-read, in L2.
constexpr int kPol = kNonTemporal;
template <int GT> struct Raw4;
template <> struct Raw4<G_F16> {
  u32x2 v;
  __device__ __forceinline__ void load(rsrc_t r, uint32_t off) { v = bload8<kPol>(r, off); }
  __device__ __forceinline__ f32x4 f32() const { return __builtin_convertvector(__builtin_bit_cast(f16x4, v), f32x4); }
};
template <> struct Raw4<G_BF16> {
  u32x2 v;
  __device__ __forceinline__ void load(rsrc_t r, uint32_t off) { v = bload8<kPol>(r, off); }
  __device__ __forceinline__ f32x4 f32() const { return __builtin_convertvector(__builtin_bit_cast(bf16x4, v), f32x4); }
};
template <> struct Raw4<G_F32> {
  u32x4 v;
  __device__ __forceinline__ void load(rsrc_t r, uint32_t off) { v = bload16<kPol>(r, off); }
  __device__ __forceinline__ f32x4 f32() const { return __builtin_bit_cast(f32x4, v); }
};

template <int GT>
__global__ __launch_bounds__(K3_THREADS, K3_OCC)
void k_decomp(const DevMat* __restrict__ mats, const Work* __restrict__ work,
              const float* __restrict__ scale, const int32_t* __restrict__ skip)
{
  const Work wi = work[xcd_remap(blockIdx.x, gridDim.x)];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  const int m = d.m, n = d.n, kpad3 = d.kpad3;
  const int m0 = wi.a, n0 = wi.b;
  const int lde = (int)d.ld_err;
  const rsrc_t re = make_rsrc(d.err, d.e_bytes);

  if (*skip != 0) {
    // zero E over the tile, 4 columns per store
    constexpr int C4 = K3_TN / 4;
    for (int idx = threadIdx.x; idx < K3_TM * C4; idx += K3_THREADS) {
      const int row = m0 + idx / C4, col = n0 + 4 * (idx % C4);
      const bool ok = row < m && col < n;
      bstore16<kPol>(u32x4{0, 0, 0, 0}, re, ok ? (uint32_t)(row * lde + col) * 4u : kOOB);
    }
    return;
  }

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int wm = wv % K3_WM, wn = wv / K3_WM;
  const int c = lane & 15, g = lane >> 4;

  // One LDS arena: the double-buffered factor stages during the products, then the finished
  // D tile (K3_TM x K3_DTP fp32) for the epilogue.
  __shared__ __attribute__((aligned(16))) char lds_raw[kLdsBytes];
  auto ldq = reinterpret_cast<uint16_t(*)[2][K3_TN][LDS_K]>(lds_raw);
  auto ldp = reinterpret_cast<uint16_t(*)[2][K3_TM][LDS_K]>(lds_raw + kStageQBytes);

  // staging: K3_TN rows of Q' and K3_TM rows of P x 32 k x {hi, lo}, in 16-byte units. The
  // operand arrays are padded with zero rows to whole tiles, so no staging load is masked.
  constexpr int QU = K3_TN * 8 / K3_THREADS, PU = K3_TM * 8 / K3_THREADS;
  static_assert(QU * K3_THREADS == K3_TN * 8 && PU * K3_THREADS == K3_TM * 8, "staging units");
  const GLOBAL uint16_t* __restrict__ q3h = gbl(d.q3_hi) + (int64_t)n0 * kpad3;
  const GLOBAL uint16_t* __restrict__ q3l = gbl(d.q3_lo) + (int64_t)n0 * kpad3;
  const GLOBAL uint16_t* __restrict__ p3h = gbl(d.p3_hi) + (int64_t)m0 * kpad3;
  const GLOBAL uint16_t* __restrict__ p3l = gbl(d.p3_lo) + (int64_t)m0 * kpad3;
  u32x4 sq[QU], sp[PU];
  // unit u of a `rows`-row operand: array (hi/lo), row, 16-byte unit; consecutive threads take
  // consecutive units of a row (coalesced global reads).
  auto unit = [](int u, int rows, int& arr, int& rr, int& q4) {
    arr = u / (rows * 4);
    const int v = u - arr * rows * 4;
    rr = v >> 2;
    q4 = v & 3;
  };
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int j = 0; j < QU; ++j) {
      int arr, rr, q4;
      unit(threadIdx.x + j * K3_THREADS, K3_TN, arr, rr, q4);
      sq[j] = *gcast<u32x4>((arr ? q3l : q3h) + (int64_t)rr * kpad3 + k0 + 8 * q4);
    }
#pragma unroll
    for (int j = 0; j < PU; ++j) {
      int arr, rr, q4;
      unit(threadIdx.x + j * K3_THREADS, K3_TM, arr, rr, q4);
      sp[j] = *gcast<u32x4>((arr ? p3l : p3h) + (int64_t)rr * kpad3 + k0 + 8 * q4);
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int j = 0; j < QU; ++j) {
      int arr, rr, q4;
      unit(threadIdx.x + j * K3_THREADS, K3_TN, arr, rr, q4);
      *reinterpret_cast<u32x4*>(&ldq[buf][arr][rr][8 * swz3(rr, q4)]) = sq[j];
    }
#pragma unroll
    for (int j = 0; j < PU; ++j) {
      int arr, rr, q4;
      unit(threadIdx.x + j * K3_THREADS, K3_TM, arr, rr, q4);
      *reinterpret_cast<u32x4*>(&ldp[buf][arr][rr][8 * swz3(rr, q4)]) = sp[j];
    }
  };

  f32x4 acc[4][4];     // [n-tile][m-tile]
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0, 0, 0, 0};

  auto compute = [&](int buf) {
    f16x8 bh[4], bl[4];
#pragma unroll
    for (int im = 0; im < 4; ++im) {
      const int rp = wm * 64 + im * 16 + c;
      bh[im] = *reinterpret_cast<const f16x8*>(&ldp[buf][0][rp][8 * swz3(rp, g)]);
      bl[im] = *reinterpret_cast<const f16x8*>(&ldp[buf][1][rp][8 * swz3(rp, g)]);
    }
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) {
      const int rq = wn * 64 + jn * 16 + c;
      const f16x8 ah = *reinterpret_cast<const f16x8*>(&ldq[buf][0][rq][8 * swz3(rq, g)]);
      const f16x8 al = *reinterpret_cast<const f16x8*>(&ldq[buf][1][rq][8 * swz3(rq, g)]);
#pragma unroll
      for (int im = 0; im < 4; ++im) {
        acc[jn][im] = mfma_f16(ah, bh[im], acc[jn][im]);
        acc[jn][im] = mfma_f16(ah, bl[im], acc[jn][im]);
        acc[jn][im] = mfma_f16(al, bh[im], acc[jn][im]);
      }
    }
  };

  const int nsteps = kpad3 / 32;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  int ks = 0;
  for (; ks + 1 < nsteps; ++ks) {
    load_stage((ks + 1) * 32);
    compute(ks & 1);
    store_stage((ks & 1) ^ 1);
    __syncthreads();
  }
  compute(ks & 1);

  // Epilogue. acc[jn][im]: lane holds D[row = m0 + wm*64 + im*16 + c][n0 + wn*64 + jn*16 + 4g
  // + {0..3}] times 2^(row exponent + column exponent). The exponents are removed and the tile
  // is written to LDS; G, E and out are then streamed in whole 128-byte lines (each wave
  // instruction covers 2 rows x 128 columns), all G/E loads issued before any is used.
  const rsrc_t rg = make_rsrc(d.grad, d.g_bytes);
  const rsrc_t ro = make_rsrc(d.out, d.out ? d.o_bytes : 0u);   // no out buffer: stores dropped
  const int ldg = (int)d.ld_grad, ldo = (int)d.ld_out;
  const GLOBAL int32_t* __restrict__ pexp = gbl(d.p3_exp);     // padded to whole tiles
  const GLOBAL int32_t* __restrict__ qexp = gbl(d.q3_exp);
  const float s = d.grad ? scale[d.block] : 0.0f;   // in-place matrices: E already holds M
  constexpr int GB = GradIO<GT>::kBytes;
  constexpr int CQ = K3_TN / 4;                      // 4-column groups per row
  constexpr int RSTEP = K3_THREADS / CQ;             // rows covered by one pass of the workgroup
  constexpr int NS = K3_TM / RSTEP;                  // passes over the tile
  static_assert(RSTEP * CQ == K3_THREADS && NS * RSTEP == K3_TM, "epilogue mapping");
  const int cq = threadIdx.x % CQ, rs = threadIdx.x / CQ;
  auto offset = [&](int st, int ld, uint32_t bytes) -> uint32_t {
    const int row = m0 + rs + RSTEP * st, col = n0 + 4 * cq;
    return (row < m && col < n) ? (uint32_t)(row * ld + col) * bytes : kOOB;
  };
  Raw4<GT> gv[NS];
  u32x4 ev[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    gv[st].load(rg, offset(st, ldg, GB));
    ev[st] = bload16<kPol>(re, offset(st, lde, 4u));
  }
  {
    int ep[4];
    u32x4 eqv[4];
#pragma unroll
    for (int im = 0; im < 4; ++im) ep[im] = pexp[m0 + wm * 64 + im * 16 + c];
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) eqv[jn] = *gcast<u32x4>(qexp + n0 + wn * 64 + jn * 16 + 4 * g);
    __syncthreads();                                  // every wave is done with the stages
    float* Dt = reinterpret_cast<float*>(lds_raw);
#pragma unroll
    for (int im = 0; im < 4; ++im)
#pragma unroll
      for (int jn = 0; jn < 4; ++jn) {
        f32x4 dv;
#pragma unroll
        for (int i = 0; i < 4; ++i) dv[i] = ldexpf(acc[jn][im][i], -(ep[im] + (int)eqv[jn][i]));
        *reinterpret_cast<f32x4*>(&Dt[(wm * 64 + im * 16 + c) * K3_DTP + wn * 64 + jn * 16 + 4 * g]) = dv;
      }
    __syncthreads();
  }
  const float* Dt = reinterpret_cast<const float*>(lds_raw);
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const f32x4 gf = gv[st].f32();
    const f32x4 ef = __builtin_bit_cast(f32x4, ev[st]);
    const f32x4 dv = *reinterpret_cast<const f32x4*>(&Dt[(rs + RSTEP * st) * K3_DTP + 4 * cq]);
    f32x4 en;
#pragma unroll
    for (int i = 0; i < 4; ++i) en[i] = __builtin_fmaf(s, gf[i], ef[i]) - dv[i];
    bstore16<kPol>(__builtin_bit_cast(u32x4, en), re, offset(st, lde, 4u));
    bstore16<kPol>(__builtin_bit_cast(u32x4, dv), ro, offset(st, ldo, 4u));
  }
}

// q <- q_next when the step is not skipped. One work item: 4096 consecutive floats of q (a
// 16-byte aligned range: q is n x r contiguous); each thread moves four 16-byte vectors, all
// loads issued before the stores.
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
  const int64_t vend = beg + ((end - beg) & ~int64_t(3));
  GLOBAL float* __restrict__ q = gbl(d.q);
  const GLOBAL float* __restrict__ qn = gbl(d.q_next);
  f32x4 v[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int64_t i = beg + 4 * ((int64_t)threadIdx.x + 256 * b);
    if (i < vend) v[b] = *gcast<f32x4>(qn + i);
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int64_t i = beg + 4 * ((int64_t)threadIdx.x + 256 * b);
    if (i < vend) *gcast<f32x4>(q + i) = v[b];
  }
  if ((int)threadIdx.x < end - vend) q[vend + threadIdx.x] = qn[vend + threadIdx.x];
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
