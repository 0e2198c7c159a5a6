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
//     one row of G (16 B of fp16) and of E (32 B), so M needs no LDS round trip. The loads go
//     through buffer descriptors: out-of-range lanes use an offset past the range and read
//     zeros, so the loop body has no branches and the next stage's loads stay in flight while
//     the current stage computes;
//   * the shared operand, Q^T split into bf16 hi/lo (prepared once per step), is staged in LDS
//     one pipeline stage (K1_KSUB x 32 columns of k) at a time, double-buffered;
//   * the flag test runs on M (one class test per element); only when a wave met a non-finite
//     M are the inputs G and E of its rows examined, after the main loop, so the flag is
//     exactly "G or E holds inf/NaN".
#include "psgd_internal.h"

#ifndef K1_RA
#define K1_RA 4      // 16-row tiles per wave
#endif
#ifndef K1_W
#define K1_W 4       // waves per workgroup
#endif
#ifndef K1_OCC
#define K1_OCC 1     // workgroups per CU the register budget is sized for
#endif
#ifndef K1_KSUB
#define K1_KSUB 2    // 32-column MFMA k groups per pipeline stage
#endif

namespace psgd {
namespace {

constexpr int K1_ROWS = K1_RA * 16 * K1_W;
constexpr int KS = 32 * K1_KSUB;       // k columns per stage
constexpr int LDS_K = KS;              // LDS row = KS bf16; 16-byte units XOR-swizzled by row
static_assert(KS == 64, "the LDS swizzle assumes 8 units per row");
// Physical 16-byte unit of logical unit q in rank row rr: with 128-byte rows, the 16 lanes of a
// read (16 consecutive rows, one unit each) and of a write (2 rows, 8 units each) hit 16
// distinct 16-byte bank groups.
__device__ __forceinline__ int swz1(int rr, int q) { return q ^ ((rr >> 1) & 7); }

template <int GT> struct Raw8;
template <> struct Raw8<G_F16> {
  u32x4 v;
  __device__ __forceinline__ void load(rsrc_t r, uint32_t off) { v = bload16(r, off); }
  __device__ __forceinline__ f32x8 f32() const { return __builtin_convertvector(__builtin_bit_cast(f16x8, v), f32x8); }
};
template <> struct Raw8<G_BF16> {
  u32x4 v;
  __device__ __forceinline__ void load(rsrc_t r, uint32_t off) { v = bload16(r, off); }
  __device__ __forceinline__ f32x8 f32() const { return __builtin_convertvector(__builtin_bit_cast(bf16x8, v), f32x8); }
};
template <> struct Raw8<G_F32> {
  u32x4 a, b;
  __device__ __forceinline__ void load(rsrc_t r, uint32_t off) { a = bload16(r, off); b = bload16(r, off + 16); }
  __device__ __forceinline__ f32x8 f32() const {
    const f32x4 x = __builtin_bit_cast(f32x4, a), y = __builtin_bit_cast(f32x4, b);
    return f32x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  }
};

struct Raw8E {
  u32x4 a, b;
  __device__ __forceinline__ void load(rsrc_t r, uint32_t off) { a = bload16(r, off); b = bload16(r, off + 16); }
  __device__ __forceinline__ f32x8 f32() const {
    const f32x4 x = __builtin_bit_cast(f32x4, a), y = __builtin_bit_cast(f32x4, b);
    return f32x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  }
};

template <int GT, int RTC>
__global__ __launch_bounds__(K1_W * kWave, K1_OCC)
void k_ef_mq(const DevMat* __restrict__ mats, const Work* __restrict__ work,
             const float* __restrict__ scale, uint8_t* __restrict__ flags)
{
  const Work wi = work[xcd_remap(blockIdx.x, gridDim.x)];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  const int m = d.m, n = d.n, npad = d.npad, rpad = d.rpad;
  const int ldg = (int)d.ld_grad, lde = (int)d.ld_err;
  const rsrc_t rg = make_rsrc(d.grad, d.g_bytes);
  const rsrc_t re = make_rsrc(d.err, d.e_bytes);
  const GLOBAL uint16_t* __restrict__ qth = gbl(d.qt_hi);
  const GLOBAL uint16_t* __restrict__ qtl = gbl(d.qt_lo);
  const float s = scale[d.block];
  constexpr int GB = GradIO<GT>::kBytes;

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int c = lane & 15, g = lane >> 4;
  const int row0 = wi.a + wv * (K1_RA * 16);
  const int rc0 = wi.b * RTC * 16;

  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][RTC * 16][LDS_K];

  // Q^T staging: RTC*16 rank rows x KS k x {hi, lo} in 16-byte units; consecutive threads take
  // consecutive units of a row (coalesced global reads). Threads past the last unit repeat it
  // (same value to the same LDS address), so the code has no branch.
  constexpr int QPR = KS / 8;                   // 16-byte units per rank row
  constexpr int UNITS = RTC * 16 * QPR * 2;
  constexpr int THREADS = K1_W * kWave;
  constexpr int UPT = (UNITS + THREADS - 1) / THREADS;
  u32x4 stage[UPT];
  auto unit = [&](int j, int& arr, int& rr, int& q) {
    int u = threadIdx.x + j * THREADS;
    u = u < UNITS ? u : UNITS - 1;
    arr = u / (RTC * 16 * QPR);
    const int rem = u - arr * (RTC * 16 * QPR);
    rr = rem / QPR;
    q = rem % QPR;
  };
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      int arr, rr, q;
      unit(j, arr, rr, q);
      stage[j] = *gcast<u32x4>((arr ? qtl : qth) + (int64_t)(rc0 + rr) * npad + k0 + 8 * q);
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      int arr, rr, q;
      unit(j, arr, rr, q);
      *reinterpret_cast<u32x4*>(&lds[buf][arr][rr][8 * swz1(rr, q)]) = stage[j];
    }
  };

  // A-fragments of one stage: row tile a, k group j -> 8 columns k0 + 32j + 8g of row
  // row0 + 16a + c. Out-of-range rows/columns read zeros.
  struct Frag { Raw8<GT> gr[K1_RA][K1_KSUB]; Raw8E er[K1_RA][K1_KSUB]; };
  auto load_m = [&](int k0, Frag& f) {
#pragma unroll
    for (int j = 0; j < K1_KSUB; ++j) {
      const int col = k0 + 32 * j + 8 * g;
#pragma unroll
      for (int a = 0; a < K1_RA; ++a) {
        const int row = row0 + a * 16 + c;
        const bool ok = row < m && col < n;
        f.gr[a][j].load(rg, ok ? (uint32_t)(row * ldg + col) * GB : kOOB);
        f.er[a][j].load(re, ok ? (uint32_t)(row * lde + col) * 4u : kOOB);
      }
    }
  };

  f32x4 acc[K1_RA][RTC];
#pragma unroll
  for (int a = 0; a < K1_RA; ++a)
#pragma unroll
    for (int cc = 0; cc < RTC; ++cc) acc[a][cc] = f32x4{0, 0, 0, 0};
  bool mbad = false;     // some M element of this lane was not finite

  auto compute = [&](int buf, const Frag& f) {
#pragma unroll
    for (int j = 0; j < K1_KSUB; ++j) {
      bf16x8 ah[K1_RA], al[K1_RA];
#pragma unroll
      for (int a = 0; a < K1_RA; ++a) {
        const f32x8 gf = f.gr[a][j].f32();
        const f32x8 ef = f.er[a][j].f32();
        f32x8 mv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          mv[e] = __builtin_fmaf(s, gf[e], ef[e]);
          mbad |= nonfinite(mv[e]);
        }
        split_bf16(mv, ah[a], al[a]);
      }
#pragma unroll
      for (int cc = 0; cc < RTC; ++cc) {
        const int pq = 8 * swz1(cc * 16 + c, 4 * j + g);
        const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&lds[buf][0][cc * 16 + c][pq]);
        const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&lds[buf][1][cc * 16 + c][pq]);
#pragma unroll
        for (int a = 0; a < K1_RA; ++a) {
          acc[a][cc] = mfma_bf16(ah[a], bh, acc[a][cc]);
          acc[a][cc] = mfma_bf16(ah[a], bl, acc[a][cc]);
          acc[a][cc] = mfma_bf16(al[a], bh, acc[a][cc]);
        }
      }
    }
  };

  const int nsteps = (npad + KS - 1) / KS;       // Q^T rows are padded to a whole stage
  Frag cur;
  load_stage(0);
  load_m(0, cur);
  store_stage(0);
  __syncthreads();
  int ks = 0;
  for (; ks + 1 < nsteps; ++ks) {
    Frag nxt;
    load_stage((ks + 1) * KS);
    load_m((ks + 1) * KS, nxt);
    compute(ks & 1, cur);
    store_stage((ks & 1) ^ 1);
    cur = nxt;
    __syncthreads();
  }
  compute(ks & 1, cur);

  // C layout of v_mfma_f32_16x16x32: lane holds rows 4g..4g+3, column c of the 16x16 tile.
  GLOBAL float* __restrict__ praw = gbl(d.p_raw);
  if (row0 + K1_RA * 16 <= m) {
#pragma unroll
    for (int a = 0; a < K1_RA; ++a)
#pragma unroll
      for (int cc = 0; cc < RTC; ++cc)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          praw[(int64_t)(row0 + a * 16 + 4 * g + i) * rpad + rc0 + cc * 16 + c] = acc[a][cc][i];
  } else {
#pragma unroll
    for (int a = 0; a < K1_RA; ++a)
#pragma unroll
      for (int cc = 0; cc < RTC; ++cc)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = row0 + a * 16 + 4 * g + i;
          if (row < m) praw[(int64_t)row * rpad + rc0 + cc * 16 + c] = acc[a][cc][i];
        }
  }

  // Flag: M non-finite somewhere in this wave's rows is rare; only then are the inputs G and
  // E of those rows examined, so the flag is exactly "G or E holds inf/NaN" (M may also be
  // non-finite through s or fp32 overflow).
  if (__builtin_amdgcn_ballot_w64(mbad) != 0) {
    bool bad = false;
    for (int col = 8 * g; col < n; col += 32) {
#pragma unroll
      for (int a = 0; a < K1_RA; ++a) {
        const int row = row0 + a * 16 + c;
        const bool ok = row < m;
        Raw8<GT> gr;
        Raw8E er;
        gr.load(rg, ok ? (uint32_t)(row * ldg + col) * GB : kOOB);
        er.load(re, ok ? (uint32_t)(row * lde + col) * 4u : kOOB);
        const f32x8 gf = gr.f32(), ef = er.f32();
#pragma unroll
        for (int e = 0; e < 8; ++e) bad |= nonfinite(gf[e]) || nonfinite(ef[e]);
      }
    }
    if (bad) flags[wi.mat] = 1;
  }
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
int ef_mq_k_per_stage() { return KS; }

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
