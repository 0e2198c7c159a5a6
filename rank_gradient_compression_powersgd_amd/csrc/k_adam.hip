// The optimizer side of the step: the global gradient norm with its clipping factor and the
// step count, and the fp32 Adam update of the uncompressed (pass-through) tensors. The update
// of the compressed matrices runs inside the decompression (k_decomp.hip), where D is formed.
//
// "Zero-Shot Text-to-Image Generation — 中文验证版", section 方法适配: Adam with gradient
// clipping and the skip rule for non-finite values. "AIGC 基本功|混合精度与数值稳定性-AMP",
// section 6.2: the global norm is taken over every gradient before clipping, and clipping
// precedes the optimizer step; section 6.1: the AdamW update. Korean summary of the paper,
// section "Mixed-Precision Training": gains, biases, embeddings and unembeddings keep 32-bit
// parameters, gradients and Adam moments.
//
// Global norm. For a compressed matrix the gradient the optimizer consumes is D = P Q'^T with
// orthonormal columns in P, so ||D||_F = ||Q'||_F: the norm is taken over q_next (n x r)
// instead of D (m x n), before D exists. Items of at most kNormItem floats are summed in fp64
// in a fixed order (deterministic), then one workgroup adds the item sums in order.
#include "psgd_internal.h"

namespace psgd {
namespace {

constexpr int kThreads = 256;

__device__ double block_sum(double v, double* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

// partial[b] = sum of x^2 over item b (fp64)
__global__ __launch_bounds__(kThreads)
void k_sqnorm(const NormItem* __restrict__ items, double* __restrict__ partial) {
  __shared__ double red[kThreads];
  const NormItem it = items[blockIdx.x];
  const float* __restrict__ p = it.ptr;
  double acc = 0.0;
  if ((reinterpret_cast<uintptr_t>(p) & 15) == 0 && (it.n & 3) == 0) {
    const int64_t n4 = it.n >> 2;
    for (int64_t i = threadIdx.x; i < n4; i += kThreads) {
      const f32x4 v = gcast<f32x4>(gbl(p))[i];
      acc += (double)v[0] * v[0] + (double)v[1] * v[1] + (double)v[2] * v[2] + (double)v[3] * v[3];
    }
  } else {
    for (int64_t i = threadIdx.x; i < it.n; i += kThreads) {
      const double x = gbl(p)[i];
      acc += x * x;
    }
  }
  const double s = block_sum(acc, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

// Sum the item sums in order; on a step that is not skipped: t += 1, norm, clipping factor.
__global__ __launch_bounds__(kThreads)
void k_adam_finalize(const double* __restrict__ partial, int n, float max_norm,
                     const int32_t* __restrict__ skip, int32_t* __restrict__ step,
                     float* __restrict__ norm_out) {
  __shared__ double red[kThreads];
  double acc = 0.0;
  for (int i = threadIdx.x; i < n; i += kThreads) acc += partial[i];
  const double total = block_sum(acc, red);
  if (threadIdx.x != 0 || *skip != 0) return;
  *step = *step + 1;
  const double norm = sqrt(total);
  const double c = (max_norm > 0.0f && norm > (double)max_norm) ? (double)max_norm / norm : 1.0;
  norm_out[0] = (float)norm;
  norm_out[1] = (float)c;
}

// fp32 AdamW over up to kAdamTensors tensors per launch; blockIdx.y selects the tensor.
__global__ __launch_bounds__(kThreads)
void k_adam_f32(AdamTensorArgs ta, AdamArgs aa, const int32_t* __restrict__ skip) {
  if (*skip != 0) return;
  const AdamTensor t = ta.t[blockIdx.y];
  const float clipf = *aa.clip;
  const float st = (float)*aa.step;
  const float rbc1 = 1.0f / (1.0f - powf(aa.beta1, st));
  const float rbc2 = 1.0f / (1.0f - powf(aa.beta2, st));
  const float omb1 = 1.0f - aa.beta1, omb2 = 1.0f - aa.beta2;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < t.n; i += stride) {
    const float g = clipf * gbl(t.grad)[i];
    const float th = gbl(t.param)[i];
    const float m1 = aa.beta1 * gbl(t.m1)[i] + omb1 * g;
    const float m2 = aa.beta2 * gbl(t.m2)[i] + omb2 * (g * g);
    const float upd = (m1 * rbc1) / (sqrtf(m2 * rbc2) + aa.eps);
    gbl(t.param)[i] = th - aa.lr * (upd + aa.weight_decay * th);
    gbl(t.m1)[i] = m1;
    gbl(t.m2)[i] = m2;
  }
}

}  // namespace

hipError_t launch_sqnorm(const NormItem* items, int n_items, double* partial, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  k_sqnorm<<<dim3(n_items), dim3(kThreads), 0, s>>>(items, partial);
  return hipGetLastError();
}

hipError_t launch_adam_finalize(const double* partial, int n, float max_norm, const int32_t* skip,
                                int32_t* step, float* norm_out, hipStream_t s) {
  k_adam_finalize<<<dim3(1), dim3(kThreads), 0, s>>>(partial, n, max_norm, skip, step, norm_out);
  return hipGetLastError();
}

hipError_t launch_adam_f32(const AdamTensor* ts, int n, const AdamArgs& aa, const int32_t* skip,
                           hipStream_t s) {
  for (int done = 0; done < n;) {
    AdamTensorArgs ta{};
    int64_t biggest = 0;
    while (done < n && ta.count < kAdamTensors) {
      ta.t[ta.count++] = ts[done];
      if (ts[done].n > biggest) biggest = ts[done].n;
      ++done;
    }
    int64_t bx = (biggest + kThreads - 1) / kThreads;
    if (bx < 1) bx = 1;
    if (bx > 1024) bx = 1024;
    k_adam_f32<<<dim3((unsigned)bx, (unsigned)ta.count), dim3(kThreads), 0, s>>>(ta, aa, skip);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace psgd
