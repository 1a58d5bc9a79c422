// h = SiLU(gate) * up in float32, re-quantised to NVFP4; and the amax of h
// for warmup calibration of its global scale.
#include "nvfp4_device.hpp"
#include "launch.hpp"

namespace nvfp4 {

// One thread per 16-element block of h (16 gate + 16 up inputs).
template <bool kBf16>
__global__ __launch_bounds__(256) void silu_requant_kernel(const void* __restrict__ gu, int64_t M,
                                                           int64_t I, int64_t ld,
                                                           const float* __restrict__ gs_ptr,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales,
                                                           uint16_t* __restrict__ dq) {
  const int64_t bpr = I / 16;
  const int64_t nblk = M * bpr;
  const float gs = *gs_ptr;
  constexpr int64_t kElem = kBf16 ? 2 : 4;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk;
       b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = b / bpr;
    const int64_t c = b - r * bpr;
    const char* row = (const char*)gu + r * ld * kElem;
    float g[16], u[16], h[16];
    load16<kBf16>(row + c * 16 * kElem, g);
    load16<kBf16>(row + (I + c * 16) * kElem, u);
#pragma unroll
    for (int i = 0; i < 16; ++i) h[i] = silu_mul(g[i], u[i]);
    uint32_t lo, hi;
    const uint32_t sq = quantize_block16(h, gs, lo, hi);
    *(uint2*)(codes + r * (I / 2) + c * 8) = make_uint2(lo, hi);
    scales[r * bpr + c] = (uint8_t)sq;
    if (dq) store_dq16(dq + r * I + c * 16, lo, hi, sq);
  }
}

template <bool kBf16>
__global__ __launch_bounds__(256) void silu_amax_kernel(const void* __restrict__ gu, int64_t M,
                                                        int64_t I, int64_t ld, float* __restrict__ partial) {
  const int64_t bpr = I / 16;
  const int64_t nblk = M * bpr;
  constexpr int64_t kElem = kBf16 ? 2 : 4;
  float m = 0.0f;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk;
       b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = b / bpr;
    const int64_t c = b - r * bpr;
    const char* row = (const char*)gu + r * ld * kElem;
    float g[16], u[16];
    load16<kBf16>(row + c * 16 * kElem, g);
    load16<kBf16>(row + (I + c * 16) * kElem, u);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(silu_mul(g[i], u[i])));
  }
  m = block_max(m);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

__global__ __launch_bounds__(256) void silu_amax_final_kernel(const float* __restrict__ partial,
                                                              int64_t n, float* __restrict__ gs_out) {
  float m = 0.0f;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) m = __builtin_fmaxf(m, partial[i]);
  m = block_max(m);
  if (threadIdx.x == 0) gs_out[0] = global_scale_from_amax(m);
}

static int64_t grid_for(int64_t nblk) {
  int64_t g = (nblk + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return g;
}

int64_t silu_amax_chunks(int64_t M, int64_t I) {
  int64_t g = grid_for(M * (I / 16));
  return g > 1024 ? 1024 : g;
}

hipError_t launch_silu_mul_requant(const void* gu, bool bf16, int64_t M, int64_t I, int64_t ld,
                                   const float* gs_h, uint8_t* codes, uint8_t* scales, uint16_t* dq,
                                   hipStream_t s) {
  const int64_t nblk = M * (I / 16);
  if (nblk == 0) return hipSuccess;
  const int64_t g = grid_for(nblk);
  if (bf16)
    hipLaunchKernelGGL(silu_requant_kernel<true>, dim3((unsigned)g), dim3(256), 0, s, gu, M, I, ld, gs_h,
                       codes, scales, dq);
  else
    hipLaunchKernelGGL(silu_requant_kernel<false>, dim3((unsigned)g), dim3(256), 0, s, gu, M, I, ld, gs_h,
                       codes, scales, dq);
  return hipGetLastError();
}

hipError_t launch_silu_mul_global_scale(const void* gu, bool bf16, int64_t M, int64_t I, int64_t ld,
                                        float* gs_out, float* partial, hipStream_t s) {
  const int64_t g = silu_amax_chunks(M, I);
  if (bf16)
    hipLaunchKernelGGL(silu_amax_kernel<true>, dim3((unsigned)g), dim3(256), 0, s, gu, M, I, ld, partial);
  else
    hipLaunchKernelGGL(silu_amax_kernel<false>, dim3((unsigned)g), dim3(256), 0, s, gu, M, I, ld, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(silu_amax_final_kernel, dim3(1), dim3(256), 0, s, partial, g, gs_out);
  return hipGetLastError();
}

}  // namespace nvfp4
