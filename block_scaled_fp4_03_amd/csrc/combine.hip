// Weighted combine of each token's k expert outputs back in token order.
#include "nvfp4_device.hpp"
#include "launch.hpp"

namespace nvfp4 {

// One thread per 8 consecutive output columns of one token: it reads the k
// permuted rows' 8-column slices (16 B of bf16 each), accumulates in slot
// order with separate float32 multiplies and adds, and writes 16 B of bf16.
template <bool kBf16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int64_t T, int k,
                                                      int64_t H, int64_t R, uint16_t* __restrict__ out) {
  const int64_t per_row = H / 8;
  const int64_t n = T * per_row;
  constexpr int64_t kElem = kBf16 ? 2 : 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / per_row;
    const int64_t c = (i - t * per_row) * 8;
    float acc[8];
    for (int j = 0; j < k; ++j) {
      int64_t row = inv[t * k + j];
      row = row < 0 ? 0 : (row >= R ? R - 1 : row);       // never leave y
      const float wj = w[t * k + j];
      float v[8];
      const char* p = (const char*)y + (row * H + c) * kElem;
      if constexpr (kBf16) {
        // each row of y is read once: non-temporal load
        typedef uint32_t u32x4n __attribute__((ext_vector_type(4)));
        const u32x4n q = __builtin_nontemporal_load((const u32x4n*)p);
        const uint32_t q4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = __uint_as_float(q4[e] << 16);
          v[2 * e + 1] = __uint_as_float(q4[e] & 0xFFFF0000u);
        }
      } else {
        const float4 a = *(const float4*)p;
        const float4 b = *(const float4*)(p + 16);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float prod = wj * v[e];
        acc[e] = j == 0 ? prod : acc[e] + prod;
      }
    }
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = (uint32_t)bf16_from_float(acc[2 * e]) | ((uint32_t)bf16_from_float(acc[2 * e + 1]) << 16);
    *(uint4*)(out + t * H + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_combine(const void* y, bool bf16, const int32_t* inv, const float* w, int64_t T, int k,
                          int64_t H, uint16_t* out, hipStream_t s) {
  const int64_t n = T * (H / 8);
  if (n == 0) return hipSuccess;
  int64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  const int64_t R = T * k;
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)g), dim3(256), 0, s, y, inv, w, T, k, H, R, out);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)g), dim3(256), 0, s, y, inv, w, T, k, H, R, out);
  return hipGetLastError();
}

}  // namespace nvfp4
