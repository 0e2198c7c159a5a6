// Small kernels: fills, uploads through kernel arguments and the skip decision.
#include <cstring>

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

// Zero `n16` 16-byte units (grid-stride, vector stores).
__global__ __launch_bounds__(256)
void k_fill_zero16(u32x4* __restrict__ p, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = u32x4{0, 0, 0, 0};
}

// Copy up to kUploadWords 32-bit words handed over as a kernel argument: a host-to-device
// upload made of kernel launches only (no copy engine, no staging buffer).
constexpr int kUploadWords = 512;
struct UploadChunk {
  uint32_t w[kUploadWords];
  int n;
};
__global__ __launch_bounds__(256)
void k_upload(uint32_t* __restrict__ dst, UploadChunk c) {
  for (int i = threadIdx.x; i < c.n; i += blockDim.x) dst[i] = c.w[i];
}

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  if ((bytes & 15) != 0 || (reinterpret_cast<uintptr_t>(p) & 15) != 0) return hipErrorInvalidValue;
  const int64_t n16 = (int64_t)(bytes / 16);
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  k_fill_zero16<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(static_cast<u32x4*>(p), n16);
  return hipGetLastError();
}

hipError_t launch_upload(void* dst, const void* src, size_t bytes, hipStream_t s) {
  if ((bytes & 3) != 0 || (reinterpret_cast<uintptr_t>(dst) & 3) != 0) return hipErrorInvalidValue;
  const uint32_t* w = static_cast<const uint32_t*>(src);
  uint32_t* d = static_cast<uint32_t*>(dst);
  size_t left = bytes / 4;
  while (left > 0) {
    UploadChunk c;
    c.n = (int)(left < (size_t)kUploadWords ? left : (size_t)kUploadWords);
    std::memcpy(c.w, w, (size_t)c.n * 4);
    k_upload<<<dim3(1), dim3(256), 0, s>>>(d, c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    w += c.n;
    d += c.n;
    left -= (size_t)c.n;
  }
  return hipSuccess;
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
