// Measurement probes: the simplest kernels that stream HBM and keep the
// matrix cores busy, so that the pipeline's achieved rates can be reported
// against what this chip reaches in practice as well as against the vendor
// peaks.  They compute nothing of the pipeline.
#include "nvfp4_device.hpp"
#include "launch.hpp"

namespace nvfp4 {

typedef uint32_t u32x4p __attribute__((ext_vector_type(4)));
typedef float floatx16p __attribute__((ext_vector_type(16)));

// Read `n16` 16-byte words once: each wave streams one contiguous chunk of
// `per_wave` words (a multiple of 1024) with sixteen 1 KiB wave-loads in
// flight, non-temporal; the words past the chunks are read grid-stride.
// Among the read patterns measured (grid-stride with 4, 8 or 16 loads in
// flight per lane; per-wave chunks with 4, 8 or 16; several sub-streams per
// wave; 1024-4096 workgroups) this one is at the top, about 10% above the
// grid-stride form.  The words are folded into one value that is stored
// only if it equals a value it cannot take in practice, so the loads are
// not removed and nothing is written.
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4p* __restrict__ p, int64_t n16,
                                                         int64_t per_wave, uint32_t* __restrict__ sink) {
  constexpr int D = 16;
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / 64);
  const int64_t w = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const u32x4p* q = p + w * per_wave + lane;
  u32x4p acc = {0u, 0u, 0u, 0u};
  for (int64_t i = 0; i < per_wave; i += 64 * D) {
    u32x4p v[D];
#pragma unroll
    for (int j = 0; j < D; ++j) v[j] = __builtin_nontemporal_load(q + i + 64 * j);
#pragma unroll
    for (int j = 0; j < D; ++j) acc ^= v[j];
  }
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = waves * per_wave + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    acc ^= __builtin_nontemporal_load(p + i);
  const uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (v == 0x9E3779B9u) sink[0] = v;
}

// Four waves per workgroup, one per SIMD; each wave runs `iters` rounds of
// eight independent v_mfma_f32_32x32x16_f16 chains.  The operands alternate
// between two sets of pseudo-random f16 values (fixed per lane), so the
// multipliers switch like they do on real data (constant operands let the
// chip clock higher than any GEMM can).  Results are stored only if they
// take a value they cannot take in practice.
__global__ __launch_bounds__(256) void mfma_probe_kernel(int64_t iters, float* __restrict__ sink) {
  const uint32_t lane = threadIdx.x & 63;
  half8_t a[2], b[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t h = (lane * 8u + j + 1u) * 0x9E3779B1u ^ (uint32_t)(s + 1) * 0x85EBCA77u ^ blockIdx.x;
      h ^= h >> 15;
      h *= 0x2C1B3C6Du;
      h ^= h >> 12;
      // values in [-2, 2) on a grid of 2^-10 and 2^-9
      const float f = (float)(int)(h & 0xFFFu) / 2048.0f - 1.0f;
      a[s][j] = (_Float16)(f * 2.0f);
      b[s][j] = (_Float16)((float)(int)((h >> 12) & 0xFFFu) / 1024.0f - 2.0f);
    }
  floatx16p acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = floatx16p{};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[c & 1], b[(c >> 1) & 1], acc[c], 0, 0, 0);
  }
  float v = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) v += acc[c][i];
  if (v == 1.2345678e30f) sink[0] = v;
}

hipError_t launch_read_probe(const void* buf, int64_t bytes, void* sink, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  // eight workgroups per compute unit, 8192 waves
  constexpr int64_t kGrid = 2048, kWaves = kGrid * 4;
  const int64_t per_wave = n16 / kWaves / 1024 * 1024;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)kGrid), dim3(256), 0, s, (const u32x4p*)buf, n16, per_wave,
                     (uint32_t*)sink);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(int64_t iters, int64_t workgroups, void* sink, hipStream_t s) {
  if (iters <= 0 || workgroups <= 0) return hipSuccess;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)workgroups), dim3(256), 0, s, iters, (float*)sink);
  return hipGetLastError();
}

}  // namespace nvfp4
