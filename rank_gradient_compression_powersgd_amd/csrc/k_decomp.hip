// K3: decompression D = P Q'^T with fp32-accurate products, and the error-feedback write-back
// E = M - D with M = s_b G + E recomputed; optional D output.
//
// "Zero-Shot Text-to-Image Generation — 中文验证版" (section 证据) asks for 32-bit products in
// the decompressed gradient. Both factors are read in fp32 (p and q_next), each row scaled by
// a power of two (computed with the factor, one exponent per row) and split into fp16 hi + lo
// (|x - hi - lo| <= 2^-22 |x|) while staged; three fp16 MFMA products (hi*hi + hi*lo + lo*hi)
// with fp32 accumulation reproduce fp32 products to about 2^-21. The power-of-two row scales
// are removed exactly with ldexp.
//
// The tile is computed transposed, D^T = Q' P^T, so the MFMA C layout gives every lane 4
// consecutive columns of one row of D. The finished tile is passed through LDS so that the
// G/E/out traffic runs in whole 128-byte lines: in the C layout one wave instruction would
// touch half of a line in each of 16 rows, which HBM serves at a markedly lower rate. G, E and
// out go through buffer descriptors: ragged edges read zeros and drop their stores in
// hardware, so the epilogue issues the loads of all its rows at once and has no branches.
//
// The workgroups of the first row of tiles also copy the q_next rows they stage into q (the
// warm start of the next step), so a non-skipped step commits q without a pass of its own.
//
// PS (ranks above one chunk): the factors arrive already scaled and split into fp16 halves
// (written once per step with the row exponents), and a stage is a plain copy into LDS. Each
// factor row is otherwise split again in every tile that uses it, about 14 conversions per
// output element at r = 896. q then comes from q_next directly, each tile of a column block
// copying its share of the block's rows, so that no row of tiles carries the whole copy.
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
// Physical unit of logical unit q in row rr (64-byte rows, 4 units): the 8 lanes an LDS pass
// serves read 8 consecutive rows, whose units land on the 8 distinct 16-byte groups of the 32
// banks (two rows per 128 bytes, four swizzle values per row parity).
__device__ __forceinline__ int swz3(int rr, int q) { return q ^ ((rr >> 1) & 3); }

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

// Adam variant of the epilogue (PT = parameter type; PT = 0 is the plain decompression). The
// decompressed gradient is consumed where it is formed instead of being written: for every
// element, g = c D (c the clipping factor), the moments m1 (bfloat16) and m2 (ue8m8: bits
// 30..15 of a non-negative float32) are updated, and the parameter takes one AdamW step
// (Zero-Shot Text-to-Image Generation — 中文验证版, section 方法适配: 16-bit Adam moments with
// gradient clipping; AIGC 基本功|混合精度与数值稳定性-AMP, section 6.1: the AdamW update).
// Per element: read G, E, theta, m1, m2; write E, theta, m1, m2 (no D).
__device__ __forceinline__ float ue8m8_to_f32(uint32_t code) { return __builtin_bit_cast(float, code << 15); }
__device__ __forceinline__ uint32_t f32_to_ue8m8(float v) {     // v >= 0; round to nearest even
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return (u + 0x3FFFu + ((u >> 15) & 1u)) >> 15;
}
template <int PT> struct ParamIO;
template <> struct ParamIO<G_F16> {
  static constexpr uint32_t kBytes = 2;
  u32x2 v;
  __device__ __forceinline__ void load(rsrc_t r, uint32_t off) { v = bload8<kPol>(r, off); }
  __device__ __forceinline__ f32x4 f32() const { return __builtin_convertvector(__builtin_bit_cast(f16x4, v), f32x4); }
  __device__ __forceinline__ static void store(f32x4 x, rsrc_t r, uint32_t off) {
    const u32x2 b = __builtin_bit_cast(u32x2, __builtin_convertvector(x, f16x4));
    __builtin_amdgcn_raw_buffer_store_b64(b, r, off, 0, kPol);
  }
};
template <> struct ParamIO<G_BF16> {
  static constexpr uint32_t kBytes = 2;
  u32x2 v;
  __device__ __forceinline__ void load(rsrc_t r, uint32_t off) { v = bload8<kPol>(r, off); }
  __device__ __forceinline__ f32x4 f32() const { return __builtin_convertvector(__builtin_bit_cast(bf16x4, v), f32x4); }
  __device__ __forceinline__ static void store(f32x4 x, rsrc_t r, uint32_t off) {
    const u32x2 b = __builtin_bit_cast(u32x2, __builtin_convertvector(x, bf16x4));
    __builtin_amdgcn_raw_buffer_store_b64(b, r, off, 0, kPol);
  }
};
template <> struct ParamIO<G_F32> {
  static constexpr uint32_t kBytes = 4;
  u32x4 v;
  __device__ __forceinline__ void load(rsrc_t r, uint32_t off) { v = bload16<kPol>(r, off); }
  __device__ __forceinline__ f32x4 f32() const { return __builtin_bit_cast(f32x4, v); }
  __device__ __forceinline__ static void store(f32x4 x, rsrc_t r, uint32_t off) {
    bstore16<kPol>(__builtin_bit_cast(u32x4, x), r, off);
  }
};

template <int GT, int PT, bool PS>
__global__ __launch_bounds__(K3_THREADS, K3_OCC)
void k_decomp(const DevMat* __restrict__ mats, const Work* __restrict__ work,
              const float* __restrict__ scale, const int32_t* __restrict__ skip, AdamArgs aa,
              int64_t* __restrict__ counters)
{
  // step counters of the plan: steps decompressed and steps skipped (one thread of the grid)
  if (counters != nullptr && blockIdx.x == 0 && threadIdx.x == 0) {
    counters[0] += 1;
    counters[1] += *skip != 0 ? 1 : 0;
  }
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

  // staging: K3_TN rows of Q' (q_next) and K3_TM rows of P (p), both fp32 with row pitch r, 32
  // ranks per stage. A group is 4 consecutive ranks of one row (one 16-byte load); 8 threads
  // cover a row's 32 ranks (one 128-byte line). Each value is scaled by its row's power of two
  // (largest entry of the row in [2^13, 2^14)) and split into fp16 hi + lo on its way into LDS.
  // Rows past n (m) and ranks past r read zeros.
  constexpr int QG = K3_TN * 8 / K3_THREADS, PG = K3_TM * 8 / K3_THREADS;
  static_assert(QG * K3_THREADS == K3_TN * 8 && PG * K3_THREADS == K3_TM * 8, "staging groups");
  const int r = d.r;
  const bool rvec = (r & 3) == 0;               // rows are whole 16-byte groups
  const rsrc_t rsq = make_rsrc(d.q_next, (uint32_t)n * (uint32_t)r * 4u);
  const rsrc_t rsp = make_rsrc(d.p, (uint32_t)m * (uint32_t)r * 4u);
  const int hq = threadIdx.x & 7, rq0 = threadIdx.x >> 3;   // group within the row, first row
  constexpr int RSTEP3 = K3_THREADS / 8;        // rows between a thread's groups
  f32x4 sq[QG], sp[PG];
  int eq[QG], epx[PG];
  uint32_t qrow[QG], prow[PG];                  // byte offsets of the thread's rows (kOOB past the end)
#pragma unroll
  for (int j = 0; j < QG; ++j) {
    const int row = n0 + rq0 + RSTEP3 * j;
    eq[j] = gbl(d.q3_exp)[row];                 // padded to whole tiles
    qrow[j] = row < n ? (uint32_t)row * (uint32_t)r * 4u : kOOB;
  }
#pragma unroll
  for (int j = 0; j < PG; ++j) {
    const int row = m0 + rq0 + RSTEP3 * j;
    epx[j] = gbl(d.p3_exp)[row];
    prow[j] = row < m ? (uint32_t)row * (uint32_t)r * 4u : kOOB;
  }
  // a row offset of kOOB stays past the buffer range (< 2 GiB) with any rank added
  auto load_group = [&](rsrc_t rs_, uint32_t rowoff, int k) -> f32x4 {
    if (rvec) return __builtin_bit_cast(f32x4, bload16(rs_, k < r ? rowoff + 4u * k : kOOB));
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = __builtin_bit_cast(float, bload4(rs_, k + e < r ? rowoff + 4u * (k + e) : kOOB));
    return v;
  };
  // split factors: a row holds kpad3 ranks as 16-byte (hi, lo) pairs per 8 ranks, so the 8
  // threads of a row read the stage's 128 bytes in order: thread hq the hi (hq even) or lo
  // half of ranks k0 + 8 (hq / 2) ..; the buffers cover whole tiles (zero rows past m, n)
  const rsrc_t rsqh = make_rsrc(d.q3h, PS ? (uint32_t)((n + K3_TN - 1) / K3_TN * K3_TN) * (uint32_t)kpad3 * 4u : 0u);
  const rsrc_t rsph = make_rsrc(d.p3h, PS ? (uint32_t)((m + K3_TM - 1) / K3_TM * K3_TM) * (uint32_t)kpad3 * 4u : 0u);
  auto load_stage = [&](int k0) {
    if constexpr (PS) {
#pragma unroll
      for (int j = 0; j < QG; ++j)
        sq[j] = __builtin_bit_cast(f32x4, bload16(rsqh, ((uint32_t)(n0 + rq0 + RSTEP3 * j) * (uint32_t)kpad3 + (uint32_t)k0) * 4u + 16u * hq));
#pragma unroll
      for (int j = 0; j < PG; ++j)
        sp[j] = __builtin_bit_cast(f32x4, bload16(rsph, ((uint32_t)(m0 + rq0 + RSTEP3 * j) * (uint32_t)kpad3 + (uint32_t)k0) * 4u + 16u * hq));
      return;
    }
    const int k = k0 + 4 * hq;
#pragma unroll
    for (int j = 0; j < QG; ++j) sq[j] = load_group(rsq, qrow[j], k);
#pragma unroll
    for (int j = 0; j < PG; ++j) sp[j] = load_group(rsp, prow[j], k);
  };
  // 4 values -> 4 fp16 hi and 4 fp16 lo at the group's place in its swizzled LDS row
  auto put_group = [&](uint16_t* hi_row, uint16_t* lo_row, int rr, f32x4 v, int ex) {
    f32x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = ldexpf(v[e], ex);
    const f16x4 h = __builtin_convertvector(x, f16x4);
    const f16x4 l = __builtin_convertvector(x - __builtin_convertvector(h, f32x4), f16x4);
    const int off = 8 * swz3(rr, hq >> 1) + 4 * (hq & 1);
    *reinterpret_cast<f16x4*>(hi_row + off) = h;
    *reinterpret_cast<f16x4*>(lo_row + off) = l;
  };
  // The first row of tiles also commits q <- q_next (the step is not skipped here): it writes
  // the fp32 groups of q_next it has just read to the same place in q.
  const bool commit = !PS && m0 == 0;
  const rsrc_t rqc = make_rsrc(d.q, commit ? (uint32_t)n * (uint32_t)r * 4u : 0u);
  auto store_stage = [&](int buf, int k0) {
    if constexpr (PS) {
      const int h = hq & 1;
#pragma unroll
      for (int j = 0; j < QG; ++j) {
        const int rr = rq0 + RSTEP3 * j;
        *reinterpret_cast<f32x4*>(&ldq[buf][h][rr][8 * swz3(rr, hq >> 1)]) = sq[j];
      }
#pragma unroll
      for (int j = 0; j < PG; ++j) {
        const int rr = rq0 + RSTEP3 * j;
        *reinterpret_cast<f32x4*>(&ldp[buf][h][rr][8 * swz3(rr, hq >> 1)]) = sp[j];
      }
      return;
    }
    const int k = k0 + 4 * hq;
#pragma unroll
    for (int j = 0; j < QG; ++j) {
      const int rr = rq0 + RSTEP3 * j;
      put_group(ldq[buf][0][rr], ldq[buf][1][rr], rr, sq[j], eq[j]);
      if (commit) {
        if (rvec) {
          bstore16(__builtin_bit_cast(u32x4, sq[j]), rqc, k < r ? qrow[j] + 4u * k : kOOB);
        } else {
          const u32x4 bits = __builtin_bit_cast(u32x4, sq[j]);
          __builtin_amdgcn_raw_buffer_store_b32(bits[0], rqc, k < r ? qrow[j] + 4u * k : kOOB, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(bits[1], rqc, k + 1 < r ? qrow[j] + 4u * (k + 1) : kOOB, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(bits[2], rqc, k + 2 < r ? qrow[j] + 4u * (k + 2) : kOOB, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(bits[3], rqc, k + 3 < r ? qrow[j] + 4u * (k + 3) : kOOB, 0, 0);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < PG; ++j) {
      const int rr = rq0 + RSTEP3 * j;
      put_group(ldp[buf][0][rr], ldp[buf][1][rr], rr, sp[j], epx[j]);
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

  if constexpr (PS) {
    // q <- q_next: the tiles of this column block share its rows, in order of their row block
    const int mt = (m + K3_TM - 1) / K3_TM, share = (K3_TN + mt - 1) / mt;
    const int rb = n0 + (m0 / K3_TM) * share;
    const int re_ = min(min(rb + share, n0 + K3_TN), n);
    if (rb < re_) {
      const GLOBAL float* __restrict__ qn = gbl(d.q_next);
      GLOBAL float* __restrict__ qc = gbl(d.q);
      const int64_t b = (int64_t)rb * r, e = (int64_t)re_ * r;
      if (rvec) {
        for (int64_t i = b / 4 + threadIdx.x; i < e / 4; i += K3_THREADS)
          *gcast<f32x4>(qc + 4 * i) = *gcast<f32x4>(qn + 4 * i);
      } else {
        for (int64_t i = b + threadIdx.x; i < e; i += K3_THREADS) qc[i] = qn[i];
      }
    }
  }
  const int nsteps = kpad3 / 32;
  load_stage(0);
  store_stage(0, 0);
  __syncthreads();
  int ks = 0;
  for (; ks + 1 < nsteps; ++ks) {
    load_stage((ks + 1) * 32);
    compute(ks & 1);
    store_stage((ks & 1) ^ 1, (ks + 1) * 32);
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
  const int erow = m0 + rs, ecol = n0 + 4 * cq;
  const bool ecolok = ecol < n;
  // byte offset of pass st in an array with leading dimension ld: a base plus st row steps
  auto offset = [&](int st, int ld, uint32_t bytes) -> uint32_t {
    const uint32_t base = ((uint32_t)erow * (uint32_t)ld + (uint32_t)ecol) * bytes;
    const uint32_t step = (uint32_t)(RSTEP * ld) * bytes;
    return (erow + RSTEP * st < m && ecolok) ? base + step * (uint32_t)st : kOOB;
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
  if constexpr (PT == 0) {
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
  } else {
    // scalars of this step: clipping factor c and the bias corrections 1 - beta^t
    const float clipf = *aa.clip;
    const float t = (float)*aa.step;
    const float rbc1 = 1.0f / (1.0f - powf(aa.beta1, t));
    const float rbc2 = 1.0f / (1.0f - powf(aa.beta2, t));
    const float omb1 = 1.0f - aa.beta1, omb2 = 1.0f - aa.beta2;
    const rsrc_t rth = make_rsrc(d.param, d.p_bytes);
    const rsrc_t rm1 = make_rsrc(d.m1, d.mo_bytes);
    const rsrc_t rm2 = make_rsrc(d.m2, d.mo_bytes);
    const int ldp = (int)d.ld_param;
    // The optimizer state is read in four quarters of the tile, each quarter's loads issued
    // while the previous quarter is updated.
    constexpr int QN = 4, HB = NS / QN;
    static_assert(HB * QN == NS, "quarters of whole passes");
    struct State { ParamIO<PT> th[HB]; u32x2 v1[HB], v2[HB]; };
    auto load_state = [&](State& S, int q) {
#pragma unroll
      for (int j = 0; j < HB; ++j) {
        const int st = q * HB + j;
        S.th[j].load(rth, offset(st, ldp, ParamIO<PT>::kBytes));
        S.v1[j] = bload8<kPol>(rm1, offset(st, n, 2u));
        S.v2[j] = bload8<kPol>(rm2, offset(st, n, 2u));
      }
    };
    auto update = [&](const State& S, int q) {
#pragma unroll
      for (int j = 0; j < HB; ++j) {
        const int st = q * HB + j;
        const f32x4 gf = gv[st].f32();
        const f32x4 ef = __builtin_bit_cast(f32x4, ev[st]);
        const f32x4 dv = *reinterpret_cast<const f32x4*>(&Dt[(rs + RSTEP * st) * K3_DTP + 4 * cq]);
        const f32x4 th0 = S.th[j].f32();
        const f32x4 m1o = __builtin_convertvector(__builtin_bit_cast(bf16x4, S.v1[j]), f32x4);
        f32x4 en, thn, m1n, m2n;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          en[i] = __builtin_fmaf(s, gf[i], ef[i]) - dv[i];
          const uint32_t code = i < 2 ? (S.v2[j][0] >> (16 * i)) & 0xFFFFu : (S.v2[j][1] >> (16 * (i - 2))) & 0xFFFFu;
          const float g = clipf * dv[i];
          m1n[i] = aa.beta1 * m1o[i] + omb1 * g;
          m2n[i] = aa.beta2 * ue8m8_to_f32(code) + omb2 * (g * g);
          const float upd = (m1n[i] * rbc1) / (sqrtf(m2n[i] * rbc2) + aa.eps);
          thn[i] = th0[i] - aa.lr * (upd + aa.weight_decay * th0[i]);
        }
        bstore16<kPol>(__builtin_bit_cast(u32x4, en), re, offset(st, lde, 4u));
        ParamIO<PT>::store(thn, rth, offset(st, ldp, ParamIO<PT>::kBytes));
        const u32x2 b1 = __builtin_bit_cast(u32x2, __builtin_convertvector(m1n, bf16x4));
        __builtin_amdgcn_raw_buffer_store_b64(b1, rm1, offset(st, n, 2u), 0, kPol);
        const u32x2 b2 = u32x2{f32_to_ue8m8(m2n[0]) | (f32_to_ue8m8(m2n[1]) << 16),
                               f32_to_ue8m8(m2n[2]) | (f32_to_ue8m8(m2n[3]) << 16)};
        __builtin_amdgcn_raw_buffer_store_b64(b2, rm2, offset(st, n, 2u), 0, kPol);
      }
    };
    State S0, S1;
    load_state(S0, 0);
    load_state(S1, 1);
    update(S0, 0);
    load_state(S0, 2);
    update(S1, 1);
    load_state(S1, 3);
    update(S0, 2);
    update(S1, 3);
  }
}

template <int GT, int PT>
hipError_t launch_gt(bool ps, dim3 grid, hipStream_t s, const DevMat* mats, const Work* work,
                     const float* scale, const int32_t* skip, const AdamArgs& aa, int64_t* counters) {
  if (ps) k_decomp<GT, PT, true><<<grid, dim3(K3_THREADS), 0, s>>>(mats, work, scale, skip, aa, counters);
  else k_decomp<GT, PT, false><<<grid, dim3(K3_THREADS), 0, s>>>(mats, work, scale, skip, aa, counters);
  return hipGetLastError();
}
template <int PT>
hipError_t launch_pt(int gt, bool ps, dim3 grid, hipStream_t s, const DevMat* mats, const Work* work,
                     const float* scale, const int32_t* skip, const AdamArgs& aa, int64_t* counters) {
  switch (gt) {
    case G_F16: return launch_gt<G_F16, PT>(ps, grid, s, mats, work, scale, skip, aa, counters);
    case G_BF16: return launch_gt<G_BF16, PT>(ps, grid, s, mats, work, scale, skip, aa, counters);
    case G_F32: return launch_gt<G_F32, PT>(ps, grid, s, mats, work, scale, skip, aa, counters);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int decomp_tile_m() { return K3_TM; }
int decomp_tile_n() { return K3_TN; }

hipError_t launch_decompress(int gt, bool presplit, const DevMat* mats, const Work* work, int n_work,
                             const float* scale, const int32_t* skip, int64_t* counters, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  return launch_pt<0>(gt, presplit, dim3(n_work), s, mats, work, scale, skip, AdamArgs{}, counters);
}

hipError_t launch_decompress_adam(int gt, int pt, bool presplit, const DevMat* mats, const Work* work, int n_work,
                                  const float* scale, const int32_t* skip, const AdamArgs& aa,
                                  int64_t* counters, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  switch (pt) {
    case G_F16: return launch_pt<G_F16>(gt, presplit, dim3(n_work), s, mats, work, scale, skip, aa, counters);
    case G_BF16: return launch_pt<G_BF16>(gt, presplit, dim3(n_work), s, mats, work, scale, skip, aa, counters);
    case G_F32: return launch_pt<G_F32>(gt, presplit, dim3(n_work), s, mats, work, scale, skip, aa, counters);
  }
  return hipErrorInvalidValue;
}

}  // namespace psgd
