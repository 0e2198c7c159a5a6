// Small kernels: fills and the skip decision.
#include "psgd_internal.h"

namespace psgd {
namespace {

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
