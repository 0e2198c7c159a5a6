// Per-resblock gradient scaling at the block boundaries of backprop.
//
// Every resblock has its own gradient scale factor S_b ("Zero-Shot Text-to-Image Generation —
// 中文验证版", section 方法适配). When backprop enters block b the incoming gradient is
// multiplied by S_b; when it leaves the block the block's output gradient is divided by S_b
// again, and Inf/NaN values are replaced by 0 there so that they do not reach other blocks
// (Korean summary of the paper, section "Mixed-Precision Training").
//
//   enter: out16[i] = to16(fp32(S_b * dx[i]))        fp16 or bf16, round to nearest even
//   exit:  dx[i] = fp32(dx[i] + fp32(g16[i] / S_b))  where g16[i] is finite, dx[i] + 0 where not;
//          *flag = 1 when any g16[i] is inf or NaN (left unchanged otherwise)
//
// The residual-stream gradient dx between blocks is fp32 in true units; inside a block it is
// 16-bit and scaled. Both kernels stream 8 elements per thread (16-byte accesses of the 16-bit
// side, two of the fp32 side) over a grid of up to 65536 workgroups. Entry loads
// non-temporally and stores plainly; exit, which rewrites the dx lines it has just read, runs
// fastest with plain loads and stores (on 81M elements: entry 83 -> 76 us, exit 184 -> 143 us
// against non-temporal accesses and an 8192-workgroup grid). The division is the correctly
// rounded IEEE one (the library is built without fast-math options), so a scale that is not a
// power of two still gives the once-rounded quotient.
#include "psgd_internal.h"

namespace psgd {
namespace {

#ifndef BS_ENTER_POL
#define BS_ENTER_POL 2   // 0: non-temporal loads and stores; 1: plain; 2: non-temporal loads, plain stores
#endif
#ifndef BS_EXIT_POL
#define BS_EXIT_POL 1
#endif
template <int POL, typename T> __device__ __forceinline__ T ld(const GLOBAL T* p) {
  if constexpr (POL == 1) return *p; else return __builtin_nontemporal_load(p);
}
template <int POL, typename T> __device__ __forceinline__ void st(T v, GLOBAL T* p) {
  if constexpr (POL == 0) __builtin_nontemporal_store(v, p); else *p = v;
}

constexpr int BS_THREADS = 256;
#ifndef BS_MAX_BLOCKS
#define BS_MAX_BLOCKS 65536    // grid-stride beyond this: 16M 8-element groups per pass
#endif

template <int DT>   // G_F16 or G_BF16: the 16-bit format inside the block
__device__ __forceinline__ u32x4 to16x8(const f32x4 a, const f32x4 b) {
  if constexpr (DT == G_F16) {
    const f16x4 ha = __builtin_convertvector(a, f16x4), hb = __builtin_convertvector(b, f16x4);
    const u32x2 ua = __builtin_bit_cast(u32x2, ha), ub = __builtin_bit_cast(u32x2, hb);
    return u32x4{ua[0], ua[1], ub[0], ub[1]};
  } else {
    const bf16x4 ha = __builtin_convertvector(a, bf16x4), hb = __builtin_convertvector(b, bf16x4);
    const u32x2 ua = __builtin_bit_cast(u32x2, ha), ub = __builtin_bit_cast(u32x2, hb);
    return u32x4{ua[0], ua[1], ub[0], ub[1]};
  }
}

// element e (0..7) of 8 packed 16-bit codes: its fp32 value and whether it is inf/NaN
template <int DT>
__device__ __forceinline__ float from16(const u32x4 w, int e, bool& nonfin) {
  const uint32_t h = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
  if constexpr (DT == G_F16) {
    nonfin = (h & 0x7C00u) == 0x7C00u;
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  } else {
    nonfin = (h & 0x7F80u) == 0x7F80u;
    return __builtin_bit_cast(float, h << 16);
  }
}

template <int DT>
__global__ __launch_bounds__(BS_THREADS)
void k_block_enter(const float* __restrict__ dx_, int64_t n, const float* __restrict__ scale,
                   uint16_t* __restrict__ out_)
{
  const GLOBAL float* dx = gbl(dx_);
  GLOBAL uint16_t* out = gbl(out_);
  const float s = *gbl(scale);
  const int64_t n8 = n >> 3;
  const int64_t stride = (int64_t)gridDim.x * BS_THREADS;
  for (int64_t i = (int64_t)blockIdx.x * BS_THREADS + threadIdx.x; i < n8; i += stride) {
    const f32x4 a = ld<BS_ENTER_POL>(gcast<f32x4>(dx + 8 * i));
    const f32x4 b = ld<BS_ENTER_POL>(gcast<f32x4>(dx + 8 * i + 4));
    st<BS_ENTER_POL>(to16x8<DT>(s * a, s * b), gcast<u32x4>(out + 8 * i));
  }
  // the last n % 8 elements, one per thread of the first workgroup
  if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
    const int64_t j = 8 * n8 + threadIdx.x;
    const float p = s * dx[j];
    if constexpr (DT == G_F16) out[j] = __builtin_bit_cast(uint16_t, (_Float16)p);
    else out[j] = __builtin_bit_cast(uint16_t, (__bf16)p);
  }
}

template <int DT>
__global__ __launch_bounds__(BS_THREADS)
void k_block_exit(float* __restrict__ dx_, const uint16_t* __restrict__ g_, int64_t n,
                  const float* __restrict__ scale, uint8_t* __restrict__ flag)
{
  GLOBAL float* dx = gbl(dx_);
  const GLOBAL uint16_t* g = gbl(g_);
  const float s = *gbl(scale);
  const int64_t n8 = n >> 3;
  const int64_t stride = (int64_t)gridDim.x * BS_THREADS;
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * BS_THREADS + threadIdx.x; i < n8; i += stride) {
    const u32x4 w = ld<BS_EXIT_POL>(gcast<u32x4>(g + 8 * i));
    f32x4 a = ld<BS_EXIT_POL>(gcast<f32x4>(dx + 8 * i));
    f32x4 b = ld<BS_EXIT_POL>(gcast<f32x4>(dx + 8 * i + 4));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bool nf0, nf1;
      const float v0 = from16<DT>(w, e, nf0), v1 = from16<DT>(w, e + 4, nf1);
      a[e] = a[e] + (nf0 ? 0.0f : v0 / s);
      b[e] = b[e] + (nf1 ? 0.0f : v1 / s);
      bad |= nf0 | nf1;
    }
    st<BS_EXIT_POL>(a, gcast<f32x4>(dx + 8 * i));
    st<BS_EXIT_POL>(b, gcast<f32x4>(dx + 8 * i + 4));
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
    const int64_t j = 8 * n8 + threadIdx.x;
    const u32x4 w = {(uint32_t)g[j], 0u, 0u, 0u};
    bool nf;
    const float v = from16<DT>(w, 0, nf);
    dx[j] = dx[j] + (nf ? 0.0f : v / s);
    bad |= nf;
  }
  // one plain store of 1 per wave that met a non-finite value (never a clear, no atomics)
  if (flag && __builtin_amdgcn_ballot_w64(bad) != 0 && (threadIdx.x & (kWave - 1)) == 0) gbl(flag)[0] = 1;
}

// Leaving block b and entering block b - 1 at the same boundary: dx = dx + g / S_b (as
// k_block_exit), then out = to16(S_{b-1} * dx) (as k_block_enter) from the new dx while it is
// in registers: 12 bytes per element instead of 10 + 6, one launch instead of two.
template <int DT>
__global__ __launch_bounds__(BS_THREADS)
void k_block_exit_enter(float* __restrict__ dx_, const uint16_t* __restrict__ g_, int64_t n,
                        const float* __restrict__ scale_exit, const float* __restrict__ scale_enter,
                        uint16_t* __restrict__ out_, uint8_t* __restrict__ flag)
{
  GLOBAL float* dx = gbl(dx_);
  const GLOBAL uint16_t* g = gbl(g_);
  GLOBAL uint16_t* out = gbl(out_);
  const float s = *gbl(scale_exit), s2 = *gbl(scale_enter);
  const int64_t n8 = n >> 3;
  const int64_t stride = (int64_t)gridDim.x * BS_THREADS;
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * BS_THREADS + threadIdx.x; i < n8; i += stride) {
    const u32x4 w = ld<BS_EXIT_POL>(gcast<u32x4>(g + 8 * i));
    f32x4 a = ld<BS_EXIT_POL>(gcast<f32x4>(dx + 8 * i));
    f32x4 b = ld<BS_EXIT_POL>(gcast<f32x4>(dx + 8 * i + 4));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bool nf0, nf1;
      const float v0 = from16<DT>(w, e, nf0), v1 = from16<DT>(w, e + 4, nf1);
      a[e] = a[e] + (nf0 ? 0.0f : v0 / s);
      b[e] = b[e] + (nf1 ? 0.0f : v1 / s);
      bad |= nf0 | nf1;
    }
    st<BS_EXIT_POL>(a, gcast<f32x4>(dx + 8 * i));
    st<BS_EXIT_POL>(b, gcast<f32x4>(dx + 8 * i + 4));
    st<BS_EXIT_POL>(to16x8<DT>(s2 * a, s2 * b), gcast<u32x4>(out + 8 * i));
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
    const int64_t j = 8 * n8 + threadIdx.x;
    const u32x4 w = {(uint32_t)g[j], 0u, 0u, 0u};
    bool nf;
    const float v = from16<DT>(w, 0, nf);
    const float x = dx[j] + (nf ? 0.0f : v / s);
    dx[j] = x;
    const float p = s2 * x;
    if constexpr (DT == G_F16) out[j] = __builtin_bit_cast(uint16_t, (_Float16)p);
    else out[j] = __builtin_bit_cast(uint16_t, (__bf16)p);
    bad |= nf;
  }
  if (flag && __builtin_amdgcn_ballot_w64(bad) != 0 && (threadIdx.x & (kWave - 1)) == 0) gbl(flag)[0] = 1;
}

int grid_for(int64_t n) {
  const int64_t groups = (n >> 3) > 0 ? (n >> 3) : 1;
  const int64_t blocks = (groups + BS_THREADS - 1) / BS_THREADS;
  return (int)(blocks < BS_MAX_BLOCKS ? blocks : BS_MAX_BLOCKS);
}

}  // namespace

hipError_t launch_block_enter(int dt, const float* dx, int64_t n, const float* scale, uint16_t* out,
                              hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const dim3 grid(grid_for(n)), block(BS_THREADS);
  if (dt == G_F16) k_block_enter<G_F16><<<grid, block, 0, s>>>(dx, n, scale, out);
  else if (dt == G_BF16) k_block_enter<G_BF16><<<grid, block, 0, s>>>(dx, n, scale, out);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_block_exit(int dt, float* dx, const uint16_t* g, int64_t n, const float* scale,
                             uint8_t* flag, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const dim3 grid(grid_for(n)), block(BS_THREADS);
  if (dt == G_F16) k_block_exit<G_F16><<<grid, block, 0, s>>>(dx, g, n, scale, flag);
  else if (dt == G_BF16) k_block_exit<G_BF16><<<grid, block, 0, s>>>(dx, g, n, scale, flag);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_block_exit_enter(int dt, float* dx, const uint16_t* g, int64_t n, const float* scale_exit,
                                   const float* scale_enter, uint16_t* out, uint8_t* flag, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const dim3 grid(grid_for(n)), block(BS_THREADS);
  if (dt == G_F16) k_block_exit_enter<G_F16><<<grid, block, 0, s>>>(dx, g, n, scale_exit, scale_enter, out, flag);
  else if (dt == G_BF16) k_block_exit_enter<G_BF16><<<grid, block, 0, s>>>(dx, g, n, scale_exit, scale_enter, out, flag);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace psgd
