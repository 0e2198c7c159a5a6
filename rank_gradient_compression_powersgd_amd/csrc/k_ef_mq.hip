// K1: fused error-feedback accumulate, P = M Q and the per-matrix non-finite flag.
//
// M = s_b * G + E is formed in fp32 registers and never stored in HBM. The error buffer and
// its finite checks come from "Zero-Shot Text-to-Image Generation — 中文验证版" (section
// 证据); the per-resblock multiplier s_b reflects per-resblock gradient scaling (same card,
// section 方法适配). The product is a tall-skinny GEMM on gfx950 MFMA
// (v_mfma_f32_16x16x32_bf16) with fp32 accumulation. Each operand is split into two bfloat16
// halves, x = hi + lo, and three products hi*hi + hi*lo + lo*hi keep the result within about
// 2^-16 of fp32 products while the kernel stays bound by HBM bandwidth.
//
// Data flow per workgroup (K1_ROWS rows of one matrix, one rank chunk), per stage of 64
// columns:
//   * G and E are read in whole 128-byte lines: 16 lanes cover one row (4 consecutive
//     elements each: 8 bytes of fp16 G, 16 bytes of E), so a wave instruction covers 4 rows.
//     (Reading the MFMA A-fragments straight from HBM would touch half a line in each of 16
//     rows per instruction, which HBM serves markedly slower.) The loads go through buffer
//     descriptors: out-of-range lanes use an offset past the range and read zeros, so the
//     loop has no branches. The next stage's loads are in flight while this stage computes;
//   * each lane forms M for its elements, tests them, splits them into bf16 hi/lo and writes
//     them to an LDS tile (rows x 64 columns, 16-byte units XOR-swizzled by row); the MFMA
//     A-fragments are read from there;
//   * the shared operand, 64 rows of q, is read in fp32, split into bf16 hi/lo and staged in
//     LDS beside it as it lies in q (one LDS row per k); the MFMA B-fragments, which need 8
//     consecutive k of one rank, come from gfx950's transposing LDS read;
//   * the flag test runs on the finished P rows: a non-finite element of M makes its row of
//     P non-finite (inf times a nonzero factor entry is inf, times zero is NaN, and NaN
//     propagates; the split of inf has a NaN low half). Only when the workgroup's P is
//     non-finite are the inputs G and E of its rows examined, after the main loop, so the
//     flag is exactly "G or E holds inf/NaN" (P may also overflow from finite inputs).
#include "psgd_internal.h"

#ifndef K1_RA
#define K1_RA 2      // 16-row MFMA tiles per wave
#endif
#ifndef K1_W
#define K1_W 4       // waves per workgroup
#endif
#ifndef K1_OCC
#define K1_OCC 2     // workgroups per CU the register budget is sized for (one converts while the other multiplies)
#endif
#define K1_KSUB 2    // 32-column MFMA k groups per pipeline stage
#ifndef K1_POLG
#define K1_POLG 0
#endif
#ifndef K1_POLE
#define K1_POLE 0
#endif

namespace psgd {
namespace {

constexpr int K1_ROWS = K1_RA * 16 * K1_W;
constexpr int K1_THREADS = K1_W * kWave;
constexpr int KS = 32 * K1_KSUB;       // k columns per stage
constexpr int LDS_K = KS;              // LDS row = KS bf16; 16-byte units XOR-swizzled by row
static_assert(KS == 64, "the LDS swizzle assumes 8 units per row");
// Physical 16-byte unit of logical unit q in row rr. The LDS serves a 16-byte read 8 lanes
// per pass over 32 four-byte banks, and every 128-byte row starts on bank 0, so an MFMA
// fragment read (8 consecutive rows from a multiple of 8, one logical unit) is conflict-free
// when those rows land on 8 distinct units: rr & 7 runs over 0..7 and rr >> 2 takes two values
// that differ only in bit 0, so XOR-ing them permutes the 8 units.
__device__ __forceinline__ int swz1(int rr, int q) { return q ^ ((rr ^ (rr >> 2)) & 7); }

// coalesced M loads: 16 lanes per row, 4 columns per lane
constexpr int LCOL = KS / 4;                    // lanes per row (16)
constexpr int LROWS = K1_THREADS / LCOL;        // rows per load step
constexpr int NST = K1_ROWS / LROWS;            // load steps per stage
static_assert(LROWS * LCOL == K1_THREADS && NST * LROWS == K1_ROWS, "load mapping");

template <int GT, int RTC>
__global__ __launch_bounds__(K1_THREADS, K1_OCC)
void k_ef_mq(const DevMat* __restrict__ mats, const Work* __restrict__ work,
             const float* __restrict__ scale, uint8_t* __restrict__ flags)
{
  const Work wi = work[xcd_remap(blockIdx.x, gridDim.x)];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  const int m = d.m, n = d.n, r = d.r, rpad = d.rpad;
  const int ldg = (int)d.ld_grad, lde = (int)d.ld_err;
  const rsrc_t rg = make_rsrc(d.grad, d.g_bytes);
  const rsrc_t re = make_rsrc(d.err, d.e_bytes);
  const rsrc_t rq = make_rsrc(d.q, (uint32_t)n * (uint32_t)r * 4u);
  const float s = d.grad ? scale[d.block] : 0.0f;   // in-place matrices: E already holds M
  constexpr int GB = GradIO<GT>::kBytes;

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int c = lane & 15, g = lane >> 4;
  const int row0 = wi.a;                        // first row of the workgroup
  const int rc0 = wi.b * RTC * 16;
  const int lu = threadIdx.x % LCOL, lr = threadIdx.x / LCOL;

  // One LDS arena: the staged operands during the main loop, the output tile afterwards.
  constexpr int RC = RTC * 16;                      // rank columns of this chunk
  constexpr int PT_LD = RC + 4;                     // output tile row (padded against bank conflicts)
  constexpr int kQBytes = 2 * KS * 128 * 2;         // q halves K-outer: KS rows of 128 ranks
  constexpr int kMBytes = 2 * K1_ROWS * LDS_K * 2;
  constexpr int kPBytes = K1_ROWS * PT_LD * 4;
  constexpr int kArena = kQBytes + kMBytes > kPBytes ? kQBytes + kMBytes : kPBytes;
  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[kArena];
  auto& ldq = *reinterpret_cast<uint16_t (*)[2][KS * 128]>(lds_raw);              // q hi, lo (K-outer)
  auto& ldm = *reinterpret_cast<uint16_t (*)[2][K1_ROWS][LDS_K]>(lds_raw + kQBytes);  // M hi, lo
  __shared__ int s_bad;

  // Warm-start staging: rows k0 .. k0 + KS - 1 of q (n x r fp32, row-major), ranks rc0 ..
  // rc0 + RC - 1, split into bf16 hi + lo and stored as they lie: LDS row k holds 128 ranks
  // (256 bytes), in 16-byte units of 8 ranks. A unit of work is 4 consecutive ranks of one row
  // (one 16-byte read of q, coalesced across consecutive threads). A B-fragment read touches
  // 32 bytes in each of the 16 rows 32 j + 8 g + 4 h + t (g, t = 0..3, h = 0, 1); XOR-ing a
  // row's unit pairs with t + 4 (g & 1) puts the 8 rows of each half-wave on 8 distinct pairs,
  // all 64 banks once. Rows past n and ranks past r read zeros; threads past the last unit
  // repeat it (same values to the same LDS addresses), so the code has no branch.
  constexpr int RG = RC / 4;                    // rank groups per row
  constexpr int QUNITS = KS * RG;
  constexpr int UPT = (QUNITS + K1_THREADS - 1) / K1_THREADS;
  const bool qvec = (r & 3) == 0;               // rows of q are whole 16-byte units
  f32x4 stq[UPT];
  auto qunit = [&](int j, int& kq, int& rg) {
    int u = threadIdx.x + j * K1_THREADS;
    u = u < QUNITS ? u : QUNITS - 1;
    kq = u / RG;
    rg = u - kq * RG;
  };
  auto swzt = [](int k, int q) { return q ^ (2 * ((k & 3) | (((k >> 3) & 1) << 2))); };
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      int kq, rg;
      qunit(j, kq, rg);
      const int rank = rc0 + 4 * rg, row = k0 + kq;
      const bool ok = row < n;
      if (qvec) {
        stq[j] = __builtin_bit_cast(f32x4, bload16(rq, ok && rank < r ? (uint32_t)(row * r + rank) * 4u : kOOB));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          stq[j][e] = __builtin_bit_cast(float, bload4(rq, ok && rank + e < r ? (uint32_t)(row * r + rank + e) * 4u : kOOB));
      }
    }
  };
  auto store_stage = [&]() {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      int kq, rg;
      qunit(j, kq, rg);
      const bf16x4 hi = __builtin_convertvector(stq[j], bf16x4);
      const bf16x4 lo = __builtin_convertvector(stq[j] - __builtin_convertvector(hi, f32x4), bf16x4);
      const int off = kq * 128 + 8 * swzt(kq, rg >> 1) + 4 * (rg & 1);
      *reinterpret_cast<bf16x4*>(&ldq[0][off]) = hi;
      *reinterpret_cast<bf16x4*>(&ldq[1][off]) = lo;
    }
  };

  // M elements of one stage: step st covers rows row0 + lr + LROWS*st, columns k0 + 4*lu + {0..3}.
  struct Raw { GradVec<GT, 4> gr[NST]; GradVec<G_F32, 4> er[NST]; };
  auto load_m = [&](int k0, Raw& f) {
    const int col = k0 + 4 * lu;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int row = row0 + lr + LROWS * st;
      const bool ok = row < m && col < n;
      f.gr[st].template load<K1_POLG>(rg, ok ? (uint32_t)(row * ldg + col) * GB : kOOB);
      f.er[st].template load<K1_POLE>(re, ok ? (uint32_t)(row * lde + col) * 4u : kOOB);
    }
  };
  auto put_m = [&](const Raw& f) {
    const int q = lu >> 1, half = lu & 1;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const f32x4 gf = f.gr[st].f32();
      const f32x4 ef = f.er[st].f32();
      f32x4 mv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mv[e] = __builtin_fmaf(s, gf[e], ef[e]);
      }
      const bf16x4 hi = __builtin_convertvector(mv, bf16x4);
      const bf16x4 lo = __builtin_convertvector(mv - __builtin_convertvector(hi, f32x4), bf16x4);
      const int rr = lr + LROWS * st;
      const int off = 8 * swz1(rr, q) + 4 * half;
      *reinterpret_cast<bf16x4*>(&ldm[0][rr][off]) = hi;
      *reinterpret_cast<bf16x4*>(&ldm[1][rr][off]) = lo;
    }
  };

  f32x4 acc[K1_RA][RTC];
#pragma unroll
  for (int a = 0; a < K1_RA; ++a)
#pragma unroll
    for (int cc = 0; cc < RTC; ++cc) acc[a][cc] = f32x4{0, 0, 0, 0};

  auto compute = [&]() {
#pragma unroll
    for (int j = 0; j < K1_KSUB; ++j) {
      bf16x8 ah[K1_RA], al[K1_RA];
#pragma unroll
      for (int a = 0; a < K1_RA; ++a) {
        const int rp = wv * (K1_RA * 16) + a * 16 + c;
        const int pq = 8 * swz1(rp, 4 * j + g);
        ah[a] = *reinterpret_cast<const bf16x8*>(&ldm[0][rp][pq]);
        al[a] = *reinterpret_cast<const bf16x8*>(&ldm[1][rp][pq]);
      }
#pragma unroll
      for (int cc = 0; cc < RTC; ++cc) {
        // ranks cc 16 .. of rows 32 j + 8 g .. + 7, in two transposing reads of 4 rows each
        // (rows k and k + 4 share their swizzle)
        const int k = 32 * j + 8 * g + (c >> 2), q = 2 * cc + ((c & 3) >> 1);
        const int off = k * 128 + 8 * swzt(k, q) + 4 * (c & 1);
        typedef short i16x4 __attribute__((ext_vector_type(4)));
        auto tr = [](const uint16_t* p) {
          return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
        };
        const bf16x8 bh = __builtin_bit_cast(bf16x8, __builtin_shufflevector(tr(&ldq[0][off]), tr(&ldq[0][off + 4 * 128]), 0, 1, 2, 3, 4, 5, 6, 7));
        const bf16x8 bl = __builtin_bit_cast(bf16x8, __builtin_shufflevector(tr(&ldq[1][off]), tr(&ldq[1][off + 4 * 128]), 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int a = 0; a < K1_RA; ++a) {
          acc[a][cc] = mfma_bf16(ah[a], bh, acc[a][cc]);
          acc[a][cc] = mfma_bf16(ah[a], bl, acc[a][cc]);
          acc[a][cc] = mfma_bf16(al[a], bh, acc[a][cc]);
        }
      }
    }
  };

  // Per stage: barrier (the previous stage's fragments are read) -> this stage into LDS ->
  // next stage's loads issued -> barrier -> MFMAs while those loads are in flight.
  const int nsteps = (n + KS - 1) / KS;
  if (threadIdx.x == 0) s_bad = 0;
  Raw cur;
  load_stage(0);
  load_m(0, cur);
  for (int ks = 0; ks < nsteps; ++ks) {
    __syncthreads();
    put_m(cur);
    store_stage();
    if (ks + 1 < nsteps) {
      load_stage((ks + 1) * KS);
      load_m((ks + 1) * KS, cur);
    }
    __syncthreads();
    compute();
  }

  // C layout of v_mfma_f32_16x16x32: lane holds rows 4g..4g+3, column c of the 16x16 tile.
  // The tile goes through LDS so that the stores to P are whole 16-byte units on consecutive
  // addresses (written straight from the C layout they would be 64-byte pieces of 4 rows).
  // They are non-temporal: scattered among the reads of G and E, writes slow the read stream
  // down well beyond their own size, and keeping them out of the caches costs it the least.
  float* pt = reinterpret_cast<float*>(lds_raw);
  __syncthreads();                              // the last stage's fragments have been read
#pragma unroll
  for (int a = 0; a < K1_RA; ++a)
#pragma unroll
    for (int cc = 0; cc < RTC; ++cc)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pt[(wv * (K1_RA * 16) + a * 16 + 4 * g + i) * PT_LD + cc * 16 + c] = acc[a][cc][i];
  __syncthreads();
  GLOBAL float* __restrict__ praw = gbl(d.p_raw);
  const int rows = min(K1_ROWS, m - row0);
  constexpr int U4 = RC / 4;                    // 16-byte units per row of the tile
  for (int u = threadIdx.x; u < rows * U4; u += K1_THREADS) {
    const int rr = u / U4, q = u - rr * U4;
    __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(&pt[rr * PT_LD + 4 * q]), gcast<f32x4>(praw + (int64_t)(row0 + rr) * rpad + rc0 + 4 * q));
  }

  // Flag: a non-finite P row in this workgroup is rare; only then are the inputs G and E of
  // its rows examined, so the flag is exactly "G or E holds inf/NaN" (P may also be
  // non-finite through s or fp32 overflow).
  bool mbad = false;
#pragma unroll
  for (int a = 0; a < K1_RA; ++a)
#pragma unroll
    for (int cc = 0; cc < RTC; ++cc)
#pragma unroll
      for (int i = 0; i < 4; ++i) mbad |= nonfinite(acc[a][cc][i]);
  if (__builtin_amdgcn_ballot_w64(mbad) != 0 && lane == 0) s_bad = 1;
  __syncthreads();
  if (s_bad != 0) {
    bool bad = false;
    for (int col = 4 * lu; col < n; col += KS) {
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const int row = row0 + lr + LROWS * st;
        const bool ok = row < m;
        GradVec<GT, 4> gr;
        GradVec<G_F32, 4> er;
        gr.load(rg, ok ? (uint32_t)(row * ldg + col) * GB : kOOB);
        er.load(re, ok ? (uint32_t)(row * lde + col) * 4u : kOOB);
        const f32x4 gf = gr.f32(), ef = er.f32();
#pragma unroll
        for (int e = 0; e < 4; ++e) bad |= nonfinite(gf[e]) || nonfinite(ef[e]);
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

hipError_t launch_ef_mq(int gt, int rtc, const DevMat* mats, const Work* work, int n_work,
                        const float* scale, uint8_t* flags, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  const dim3 grid(n_work), block(K1_THREADS);
  switch (gt) {
    case G_F16: return launch_gt<G_F16>(rtc, grid, block, s, mats, work, scale, flags);
    case G_BF16: return launch_gt<G_BF16>(rtc, grid, block, s, mats, work, scale, flags);
    case G_F32: return launch_gt<G_F32>(rtc, grid, block, s, mats, work, scale, flags);
  }
  return hipErrorInvalidValue;
}

}  // namespace psgd
