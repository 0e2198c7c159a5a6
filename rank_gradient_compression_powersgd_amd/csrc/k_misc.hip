// Small kernels: warm-start operand preparation, fills and the skip decision.
#include "psgd_internal.h"

namespace psgd {
namespace {

// q (n x r fp32, caller layout) -> q^T split into bf16 hi + lo (rpad x npad), the shared
// operand of K1. One 32 x 32 tile per block, transposed through LDS.
__global__ __launch_bounds__(256)
void k_prep_qt(const DevMat* __restrict__ mats, const Work* __restrict__ work)
{
  const Work wi = work[blockIdx.x];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  const int n = d.n, r = d.r, rpad = d.rpad, npad = d.npad;
  const int n0 = wi.a, r0 = wi.b;
  __shared__ float tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int nn = n0 + ty + 8 * j, rr = r0 + tx;
    tile[ty + 8 * j][tx] = (nn < n && rr < r) ? gbl(d.q)[(int64_t)nn * r + rr] : 0.0f;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rr = r0 + ty + 8 * j, nn = n0 + tx;
    if (rr < rpad && nn < npad) {
      const float x = tile[tx][ty + 8 * j];
      const __bf16 h = (__bf16)x;
      gbl(d.qt_hi)[(int64_t)rr * npad + nn] = bf16_bits(h);
      gbl(d.qt_lo)[(int64_t)rr * npad + nn] = bf16_bits((__bf16)(x - (float)h));
    }
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
