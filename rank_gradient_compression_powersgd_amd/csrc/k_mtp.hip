// K2: Q' = M^T P, the next warm start, with M = s_b G + E recomputed from G and E.
//
// The factor product comes from the P·Q decomposition of the Korean summary of the DALL·E
// paper (section "Distributed Optimization"). The contraction runs over the m rows of M, so an
// MFMA B-fragment needs 8 consecutive rows of one column. Reading that directly would
// stride through memory. Instead every lane loads an 8-row x TC-column block of M: each load
// is TC consecutive columns of one row, and a wave instruction covers 4 rows x 16 TC columns,
// contiguous along the row. The lane then holds the B-fragments of TC column tiles at once.
// Column tile t of a wave holds columns {TC j + t : j = 0..15} of its 16 TC-column strip.
// The shared operand P^T, split into bf16 hi/lo by the orthonormalisation kernel, is staged
// in LDS 32 rows of m at a time and double-buffered. Products use the same three-term bf16
// split as K1. G and E are read through buffer descriptors (out-of-range reads give zeros),
// so the loop body has no branches and the next rows' loads overlap the current MFMAs.
//
// Epilogue: Q' is written in fp32 (the caller's q_next). When the whole rank fits one chunk
// the kernel also writes each row's exponent for the decompression: the power of two that
// brings the row's largest entry into [2^13, 2^14) before the decompression splits it.
#include "psgd_internal.h"

namespace psgd {
namespace {

// Eight waves of two column tiles (256 columns per workgroup) with one 32-row k group per
// stage keep each wave at 188 VGPRs, so a CU holds two waves per SIMD; four waves of four
// tiles (two k groups) needed 422 registers and ran one wave per SIMD, 1.89 -> 1.80 ms on the
// 64-resblock rank-112 shard (the accumulators shrink with TC, and the second wave per SIMD
// covers the loads of the first).
#ifndef K2_W
#define K2_W 8       // waves per workgroup
#endif
#ifndef K2_TC
#define K2_TC 2      // consecutive columns per lane = column tiles per wave (2 or 4)
#endif
#ifndef K2_POLG
#define K2_POLG 0
#endif
#ifndef K2_POLE
#define K2_POLE 0
#endif
#ifndef K2_OCC
#define K2_OCC 1     // workgroups per CU the register budget is sized for
#endif
#ifndef K2_KSUB
#define K2_KSUB 1    // 32-row MFMA k groups per pipeline stage (rows of M in flight per stage)
#endif
constexpr int KR = 32 * K2_KSUB;          // rows of M per stage
constexpr int LDS_K = KR;                 // LDS row = KR bf16, 16-byte units XOR-swizzled
constexpr int UPR = KR / 8;               // 16-byte units per LDS row
// Physical unit of logical unit q in row rr. The LDS serves a 16-byte read 8 lanes per pass
// over 32 four-byte banks (128 bytes), so the 8 consecutive rows a fragment read takes in one
// pass must land on 8 distinct 16-byte groups: with 64-byte rows, rr & 1 picks the half of the
// 128 bytes and (rr >> 1) & 3 the unit in it; with 128-byte rows, the low 3 bits of rr do.
__device__ __forceinline__ int swz2(int rr, int q) {
  if constexpr (UPR == 4) return q ^ ((rr >> 1) & 3);
  else return q ^ (rr & 7);
}
static_assert(UPR == 4 || UPR == 8, "stage of 32 or 64 rows");
constexpr int TC = K2_TC;
constexpr int WCOLS = 16 * TC;            // columns per wave

template <int GT, int RTC>
__global__ __launch_bounds__(K2_W * kWave, K2_OCC)
void k_mtp(const DevMat* __restrict__ mats, const Work* __restrict__ work,
           const float* __restrict__ scale)
{
  const Work wi = work[xcd_remap(blockIdx.x, gridDim.x)];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  const int m = d.m, n = d.n, mpad = d.mpad, r = d.r, rpad = d.rpad;
  const int ldg = (int)d.ld_grad, lde = (int)d.ld_err;
  const rsrc_t rg = make_rsrc(d.grad, d.g_bytes);
  const rsrc_t re = make_rsrc(d.err, d.e_bytes);
  const GLOBAL uint16_t* __restrict__ pth = gbl(d.pt_hi);
  const GLOBAL uint16_t* __restrict__ ptl = gbl(d.pt_lo);
  const float s = d.grad ? scale[d.block] : 0.0f;   // in-place matrices: E already holds M
  constexpr int GB = GradIO<GT>::kBytes;

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int c = lane & 15, g = lane >> 4;
  const int colbase = wi.a + wv * WCOLS + TC * c;
  const bool colok = colbase < n;              // n % 8 == 0: TC-column groups are all in or out
  const int rc0 = wi.b * RTC * 16;

  // One LDS arena: the staged P^T during the main loop, the output tile afterwards.
  constexpr int RC = RTC * 16;                  // rank columns of this chunk
  constexpr int QT_LD = RC + 4;                 // output tile row (padded against bank conflicts)
  constexpr int kSBytes = 2 * 2 * RC * LDS_K * 2;
  constexpr int kTBytes = K2_W * WCOLS * QT_LD * 4;
  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[kSBytes > kTBytes ? kSBytes : kTBytes];
  __shared__ int s_ex[K2_W * WCOLS];
  auto& lds = *reinterpret_cast<uint16_t (*)[2][2][RC][LDS_K]>(lds_raw);

  // P^T staging: RTC*16 rank rows x KR m x {hi, lo}; threads past the last unit repeat it.
  constexpr int UNITS = RTC * 16 * UPR * 2;
  constexpr int THREADS = K2_W * kWave;
  constexpr int UPT = (UNITS + THREADS - 1) / THREADS;
  u32x4 stage[UPT];
  // consecutive threads take consecutive units of a row; threads past the last unit repeat it
  auto unit = [&](int j, int& arr, int& rr, int& q4) {
    int u = threadIdx.x + j * THREADS;
    u = u < UNITS ? u : UNITS - 1;
    arr = u / (RTC * 16 * UPR);
    const int rem = u - arr * (RTC * 16 * UPR);
    rr = rem / UPR;
    q4 = rem % UPR;
  };
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      int arr, rr, q4;
      unit(j, arr, rr, q4);
      stage[j] = *gcast<u32x4>((arr ? ptl : pth) + (int64_t)(rc0 + rr) * mpad + k0 + 8 * q4);
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      int arr, rr, q4;
      unit(j, arr, rr, q4);
      *reinterpret_cast<u32x4*>(&lds[buf][arr][rr][8 * swz2(rr, q4)]) = stage[j];
    }
  };

  // sub-stage j: 8 rows k0 + 32j + 8g + kk, TC columns colbase..; out-of-range reads give zeros.
  struct Frag { GradVec<GT, TC> gr[K2_KSUB][8]; GradVec<G_F32, TC> er[K2_KSUB][8]; };
  auto load_m = [&](int k0, Frag& f) {
#pragma unroll
    for (int j = 0; j < K2_KSUB; ++j)
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int row = k0 + 32 * j + 8 * g + kk;
        const bool ok = colok && row < m;
        f.gr[j][kk].template load<K2_POLG>(rg, ok ? (uint32_t)(row * ldg + colbase) * GB : kOOB);
        f.er[j][kk].template load<K2_POLE>(re, ok ? (uint32_t)(row * lde + colbase) * 4u : kOOB);
      }
  };

  f32x4 acc[RTC][TC];
#pragma unroll
  for (int i = 0; i < RTC; ++i)
#pragma unroll
    for (int t = 0; t < TC; ++t) acc[i][t] = f32x4{0, 0, 0, 0};

  auto compute = [&](int buf, const Frag& f) {
#pragma unroll
    for (int j = 0; j < K2_KSUB; ++j) {
      // B-fragments: tile t takes column t of every loaded row (k = 32j + 8g + kk).
      f32x8 mt[TC];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const auto gf = f.gr[j][kk].f32();
        const auto ef = f.er[j][kk].f32();
#pragma unroll
        for (int t = 0; t < TC; ++t) mt[t][kk] = __builtin_fmaf(s, gf[t], ef[t]);
      }
      bf16x8 bh[TC], bl[TC];
#pragma unroll
      for (int t = 0; t < TC; ++t) split_bf16(mt[t], bh[t], bl[t]);
#pragma unroll
      for (int i = 0; i < RTC; ++i) {
        const int pq = 8 * swz2(i * 16 + c, 4 * j + g);
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&lds[buf][0][i * 16 + c][pq]);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(&lds[buf][1][i * 16 + c][pq]);
#pragma unroll
        for (int t = 0; t < TC; ++t) {
          acc[i][t] = mfma_bf16(ah, bh[t], acc[i][t]);
          acc[i][t] = mfma_bf16(ah, bl[t], acc[i][t]);
          acc[i][t] = mfma_bf16(al, bh[t], acc[i][t]);
        }
      }
    }
  };

  const int nsteps = mpad / KR;                // P^T columns are padded to a whole stage
  Frag cur;
  load_stage(0);
  load_m(0, cur);
  store_stage(0);
  __syncthreads();
  int ks = 0;
  for (; ks + 1 < nsteps; ++ks) {
    Frag nxt;
    load_stage((ks + 1) * KR);
    load_m((ks + 1) * KR, nxt);
    compute(ks & 1, cur);
    store_stage((ks & 1) ^ 1);
    cur = nxt;
    __syncthreads();
  }
  compute(ks & 1, cur);

  // Output tile (i, t): lane holds Q'^T rows rc0 + 16i + 4g + {0..3}, i.e. Q'[colbase + t][..].
  // The tile goes through LDS so that the stores to Q' are whole 16-byte units on consecutive
  // addresses (from the C layout they would be 64-byte pieces of 16 rows), stored
  // non-temporally as in the M Q kernel.
  float* qt = reinterpret_cast<float*>(lds_raw);          // [K2_W * WCOLS][QT_LD]
  const bool whole = RC == rpad;                // this chunk covers the whole padded rank
  __syncthreads();                              // the staged P^T has been read
#pragma unroll
  for (int t = 0; t < TC; ++t) {
    const int lc = wv * WCOLS + TC * c + t;     // column of the workgroup's block
#pragma unroll
    for (int i = 0; i < RTC; ++i)
      *reinterpret_cast<f32x4*>(&qt[lc * QT_LD + i * 16 + 4 * g]) = acc[i][t];
    if (whole) {
      // Row exponent of the decompression operand: the power of two that brings the row's
      // largest entry into [2^13, 2^14) before its fp16 split.
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < RTC; ++i)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) amax = fmaxf(amax, fabsf(acc[i][t][ii]));
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      if (g == 0) s_ex[lc] = fp16_row_exponent(amax);
    }
  }
  __syncthreads();

  constexpr int THREADS_ = K2_W * kWave;
  const int ncols = min(K2_W * WCOLS, n - wi.a);          // rows of Q' this workgroup owns
  const int rend = min(r, rc0 + RC);
  GLOBAL float* __restrict__ qn = gbl(d.q_next);
  if ((r & 3) == 0) {
    const int U4 = (rend - rc0) / 4;            // 16-byte units per row
    for (int u = threadIdx.x; u < ncols * U4; u += THREADS_) {
      const int j = u / U4, q = u - j * U4;
      __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(&qt[j * QT_LD + 4 * q]), gcast<f32x4>(qn + (int64_t)(wi.a + j) * r + rc0 + 4 * q));
    }
  } else {
    const int w = rend - rc0;
    for (int u = threadIdx.x; u < ncols * w; u += THREADS_) {
      const int j = u / w, q = u - j * w;
      qn[(int64_t)(wi.a + j) * r + rc0 + q] = qt[j * QT_LD + q];
    }
  }
  if (!whole) return;

  GLOBAL int32_t* __restrict__ q3e = gbl(d.q3_exp);
  for (int j = threadIdx.x; j < ncols; j += THREADS_) q3e[wi.a + j] = s_ex[j];
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

int mtp_cols_per_block() { return K2_W * WCOLS; }
int mtp_rows_per_stage() { return KR; }

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
