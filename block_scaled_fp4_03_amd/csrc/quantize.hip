// NVFP4 quantisation of float tensors and global-scale (amax) reductions.
#include <mutex>

#include "nvfp4_device.hpp"
#include "launch.hpp"

namespace nvfp4 {

// One thread per 16-element block.  Consecutive threads take consecutive
// blocks of a row, so a wave reads 1-2 KB of contiguous input and writes
// 512 B of codes and 64 B of scales contiguously: the op is an HBM stream.
template <bool kBf16>
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ x, int64_t rows,
                                                       int64_t blocks_per_row, int64_t ld_x,
                                                       const float* __restrict__ gs_ptr,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales,
                                                       uint16_t* __restrict__ dq) {
  const int64_t nblk = rows * blocks_per_row;
  const float gs = *gs_ptr;
  constexpr int64_t kElem = kBf16 ? 2 : 4;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk;
       b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = b / blocks_per_row;
    const int64_t c = b - r * blocks_per_row;
    float v[16];
    load16<kBf16>((const char*)x + (r * ld_x + c * 16) * kElem, v);
    uint32_t lo, hi;
    const uint32_t sq = quantize_block16(v, gs, lo, hi);
    *(uint2*)(codes + b * 8) = make_uint2(lo, hi);
    scales[b] = (uint8_t)sq;
    if (dq) store_dq16(dq + b * 16, lo, hi, sq);
  }
}

// Stage 1 of the amax reduction: block (c, b) takes the max of |x| over a
// contiguous chunk of slice b and writes it to partial[b * chunks + c].
// Max is exact and order-independent, so the result does not depend on the
// launch shape.
template <bool kBf16>
__global__ __launch_bounds__(256) void amax_partial_kernel(const void* __restrict__ x, int64_t n,
                                                           int64_t stride, int64_t chunk,
                                                           float* __restrict__ partial) {
  const int64_t b = blockIdx.y;
  const int64_t c = blockIdx.x;
  const int64_t lo = c * chunk;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  constexpr int64_t kElem = kBf16 ? 2 : 4;
  const char* base = (const char*)x + b * stride * kElem;
  float m = 0.0f;
  // 8 elements per thread-step (16 B for bf16, 32 B for f32); n % 8 == 0.
  for (int64_t i = lo + (int64_t)threadIdx.x * 8; i < hi; i += (int64_t)blockDim.x * 8) {
    if constexpr (kBf16) {
      const uint4 q = *(const uint4*)(base + i * 2);
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        m = __builtin_fmaxf(m, __builtin_fabsf(__uint_as_float(w[j] << 16)));
        m = __builtin_fmaxf(m, __builtin_fabsf(__uint_as_float(w[j] & 0xFFFF0000u)));
      }
    } else {
      const float4 a = *(const float4*)(base + i * 4);
      const float4 d = *(const float4*)(base + i * 4 + 16);
      m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(a.x), __builtin_fabsf(a.y)),
                                             __builtin_fmaxf(__builtin_fabsf(a.z), __builtin_fabsf(a.w))));
      m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(d.x), __builtin_fabsf(d.y)),
                                             __builtin_fmaxf(__builtin_fabsf(d.z), __builtin_fabsf(d.w))));
    }
  }
  m = block_max(m);
  if (threadIdx.x == 0) partial[b * gridDim.x + c] = m;
}

// Stage 2: one block per slice folds the partial maxima into a global scale.
__global__ __launch_bounds__(256) void amax_final_kernel(const float* __restrict__ partial,
                                                         int64_t chunks, float* __restrict__ gs_out) {
  const int64_t b = blockIdx.x;
  float m = 0.0f;
  for (int64_t i = threadIdx.x; i < chunks; i += blockDim.x)
    m = __builtin_fmaxf(m, partial[b * chunks + i]);
  m = block_max(m);
  if (threadIdx.x == 0) gs_out[b] = global_scale_from_amax(m);
}

// Scratch memory of the no-allocation global-scale entry point: the partial
// maxima of launch_global_scale, kNoAllocScratchFloats floats per device,
// held from the library's load to the end of the process.  In host code
// `scratch` names a host-side stand-in, never the device copy: the device
// address is looked up once per device with hipGetSymbolAddress and only
// that address is passed to kernels.
static __device__ __align__(256) float scratch[kNoAllocScratchFloats];

namespace {
constexpr int kMaxDevices = 64;
float* g_scratch_ptr[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(float** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  // once per device, with that device current (it is: dev is the current one)
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? (float*)p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return *ptr ? hipSuccess : hipErrorInvalidSymbol;
}

int64_t amax_chunks(int64_t n) {
  // about 64 KiB of input per block, at most 1024 blocks per slice
  int64_t c = (n + 16383) / 16384;
  if (c < 1) c = 1;
  if (c > 1024) c = 1024;
  return c;
}

hipError_t launch_quantize(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld_x,
                           const float* gs, uint8_t* codes, uint8_t* scales, uint16_t* dq, hipStream_t s) {
  const int64_t bpr = cols / 16;
  const int64_t nblk = rows * bpr;
  if (nblk == 0) return hipSuccess;
  int64_t grid = (nblk + 255) / 256;
  if (grid > 65536) grid = 65536;
  if (bf16)
    hipLaunchKernelGGL(quantize_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, x, rows, bpr,
                       ld_x, gs, codes, scales, dq);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, x, rows, bpr,
                       ld_x, gs, codes, scales, dq);
  return hipGetLastError();
}

hipError_t launch_global_scale(const void* x, bool bf16, int64_t batch, int64_t n, int64_t stride,
                               float* gs_out, float* partial, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  const int64_t chunks = amax_chunks(n);
  const int64_t chunk = ((n + chunks - 1) / chunks + 7) / 8 * 8;
  if (bf16)
    hipLaunchKernelGGL(amax_partial_kernel<true>, dim3((unsigned)chunks, (unsigned)batch), dim3(256), 0,
                       s, x, n, stride, chunk, partial);
  else
    hipLaunchKernelGGL(amax_partial_kernel<false>, dim3((unsigned)chunks, (unsigned)batch), dim3(256), 0,
                       s, x, n, stride, chunk, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(amax_final_kernel, dim3((unsigned)batch), dim3(256), 0, s, partial, chunks, gs_out);
  return hipGetLastError();
}

}  // namespace nvfp4
