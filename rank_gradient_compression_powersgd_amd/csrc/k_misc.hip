// Small kernels: warm-start operand preparation, fills and the skip decision.
#include "psgd_internal.h"

namespace psgd {
namespace {

// q (n x r fp32, caller layout) -> q^T split into bf16 hi + lo (rpad x npad), the shared
// operand of K1. One work item: 64 rows [a, a + 64) of q. They are staged in LDS 128 rank
// columns at a time (coalesced loads along q's rows), then written as rank rows: each thread
// stores 8 consecutive columns of q^T (16 bytes of hi and of lo). Rank columns at or beyond r
// read as zero. Columns of q^T at or beyond n are never written (they stay zero).
constexpr int PQ_N = 64;
constexpr int PQ_R = 128;
__global__ __launch_bounds__(256)
void k_prep_qt(const DevMat* __restrict__ mats, const Work* __restrict__ work)
{
  const Work wi = work[blockIdx.x];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  const int n = d.n, r = d.r, rpad = d.rpad, npad = d.npad;
  const int n0 = wi.a;
  const bool vec = (r & 3) == 0;
  const GLOBAL float* __restrict__ q = gbl(d.q);
  GLOBAL uint16_t* __restrict__ qth = gbl(d.qt_hi);
  GLOBAL uint16_t* __restrict__ qtl = gbl(d.qt_lo);
  __shared__ float tile[PQ_N][PQ_R + 1];
  for (int rc0 = 0; rc0 < rpad; rc0 += PQ_R) {
    const int rw = min(PQ_R, rpad - rc0);
    if (vec) {
      const int u4 = rw / 4;
      for (int idx = threadIdx.x; idx < PQ_N * u4; idx += 256) {
        const int j = idx / u4, k = (idx - j * u4) * 4;
        f32x4 v = f32x4{0, 0, 0, 0};
        if (n0 + j < n && rc0 + k < r) v = *gcast<f32x4>(q + (int64_t)(n0 + j) * r + rc0 + k);
#pragma unroll
        for (int e = 0; e < 4; ++e) tile[j][k + e] = v[e];
      }
    } else {
      for (int idx = threadIdx.x; idx < PQ_N * rw; idx += 256) {
        const int j = idx / rw, k = idx - j * rw;
        tile[j][k] = (n0 + j < n && rc0 + k < r) ? q[(int64_t)(n0 + j) * r + rc0 + k] : 0.0f;
      }
    }
    __syncthreads();
    for (int u = threadIdx.x; u < rw * (PQ_N / 8); u += 256) {
      const int rr = u / (PQ_N / 8), j8 = (u % (PQ_N / 8)) * 8;
      if (n0 + j8 >= n) continue;                       // n % 8 == 0: whole units in or out
      uint32_t h[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = tile[j8 + 2 * e][rr], x1 = tile[j8 + 2 * e + 1][rr];
        const __bf16 h0 = (__bf16)x0, h1 = (__bf16)x1;
        h[e] = bf16_bits(h0) | ((uint32_t)bf16_bits(h1) << 16);
        l[e] = bf16_bits((__bf16)(x0 - (float)h0)) | ((uint32_t)bf16_bits((__bf16)(x1 - (float)h1)) << 16);
      }
      *gcast<u32x4>(qth + (int64_t)(rc0 + rr) * npad + n0 + j8) = u32x4{h[0], h[1], h[2], h[3]};
      *gcast<u32x4>(qtl + (int64_t)(rc0 + rr) * npad + n0 + j8) = u32x4{l[0], l[1], l[2], l[3]};
    }
    __syncthreads();
  }
}

__global__ void k_zero_u8(uint8_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ void k_zero_i32(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

constexpr int kPassPerLaunch = 32;
struct PassArgs {
  const float* ptr[kPassPerLaunch];
  int64_t n[kPassPerLaunch];
  int count;
};

// skip |= any flag | any non-finite scale | any non-finite pass-through element
__global__ __launch_bounds__(256)
void k_check_finite(const uint8_t* __restrict__ flags, int n_flags,
                    const float* __restrict__ scale, int n_scale, PassArgs pa,
                    int32_t* __restrict__ skip)
{
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  bool bad = false;
  if (flags)
    for (int64_t i = tid; i < n_flags; i += stride) bad |= flags[i] != 0;
  if (scale)
    for (int64_t i = tid; i < n_scale; i += stride) bad |= nonfinite(scale[i]);
  for (int t = 0; t < pa.count; ++t) {
    const float* p = pa.ptr[t];
    const int64_t nn = pa.n[t];
    for (int64_t i = tid; i < nn; i += stride) bad |= nonfinite(p[i]);
  }
  if (bad) *skip = 1;
}

}  // namespace

hipError_t launch_prep_qt(const DevMat* mats, const Work* work, int n_work, int, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  k_prep_qt<<<dim3(n_work), dim3(256), 0, s>>>(mats, work);
  return hipGetLastError();
}

hipError_t launch_zero_u8(uint8_t* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_zero_u8<<<dim3((n + 255) / 256), dim3(256), 0, s>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_zero_i32<<<dim3((n + 255) / 256), dim3(256), 0, s>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_check_finite(const uint8_t* flags, int n_flags, const float* scale, int n_scale,
                               const float* const* pass_ptr, const int64_t* pass_n, int n_pass,
                               int32_t* skip, hipStream_t s) {
  int done = 0;
  bool first = true;
  while (first || done < n_pass) {
    PassArgs pa{};
    pa.count = 0;
    int64_t biggest = first ? (n_flags > n_scale ? n_flags : n_scale) : 0;
    while (done < n_pass && pa.count < kPassPerLaunch) {
      pa.ptr[pa.count] = pass_ptr[done];
      pa.n[pa.count] = pass_n[done];
      if (pass_n[done] > biggest) biggest = pass_n[done];
      ++pa.count;
      ++done;
    }
    int64_t blocks = (biggest + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 1024) blocks = 1024;
    k_check_finite<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
        first ? flags : nullptr, n_flags, first ? scale : nullptr, n_scale, pa, skip);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    first = false;
  }
  return hipSuccess;
}

}  // namespace psgd
