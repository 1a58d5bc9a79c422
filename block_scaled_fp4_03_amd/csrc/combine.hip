// Weighted combine of each token's k expert outputs back in token order,
// with an optional residual added before the one rounding to bf16.
#include "nvfp4_device.hpp"
#include "launch.hpp"

namespace nvfp4 {

// One thread per 8 consecutive output columns of one token: it reads the k
// permuted rows' 8-column slices (16 B of bf16 each), accumulates in slot
// order with separate float32 multiplies and adds, and writes 16 B of bf16.
// The slot indices, weights and row slices are all requested before the
// first product (KMAX slots unrolled, those past k skipped), so a thread
// waits for two memory round trips, not two per slot.  With a residual (bf16
// [T, H]), its 8 values are loaded with the slices and added to the slot sum
// as one more float32 addition.
// The grid is (column blocks, tokens) when T fits the grid's y extent: the
// token is the workgroup's, so its slot indices and weights are uniform
// loads, and there is no division per thread; else one dimension, strided.
template <bool kBf16, int KMAX, bool kGrid2D>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int64_t T, int k,
                                                      int64_t H, int64_t R,
                                                      const uint16_t* __restrict__ residual,
                                                      uint16_t* __restrict__ out) {
  const int64_t per_row = H / 8;
  const int64_t n = kGrid2D ? per_row : T * per_row;
  constexpr int64_t kElem = kBf16 ? 2 : 4;
  typedef uint32_t u32x4n __attribute__((ext_vector_type(4)));
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = kGrid2D ? (int64_t)blockIdx.y : i / per_row;
    const int64_t c = (kGrid2D ? i : i - t * per_row) * 8;
    int64_t row[KMAX];
    float wj[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        const int64_t r = inv[t * k + j];
        row[j] = r < 0 ? 0 : (r >= R ? R - 1 : r);       // never leave y
        wj[j] = w[t * k + j];
      } else {
        row[j] = 0;
        wj[j] = 0.0f;
      }
    }
    // the slices stay in their stored form until their turn in the sum
    u32x4n q[KMAX][kBf16 ? 1 : 2];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j >= k) continue;
      const char* p = (const char*)y + (row[j] * H + c) * kElem;
      if constexpr (kBf16) {
        q[j][0] = __builtin_nontemporal_load((const u32x4n*)p);   // each row of y is read once
      } else {
        q[j][0] = *(const u32x4n*)p;
        q[j][1] = *(const u32x4n*)(p + 16);
      }
    }
    u32x4n rq = {0u, 0u, 0u, 0u};
    if (residual) rq = __builtin_nontemporal_load((const u32x4n*)(residual + t * H + c));
    float acc[8];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j >= k) continue;
      float v[8];
      if constexpr (kBf16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = __uint_as_float(q[j][0][e] << 16);
          v[2 * e + 1] = __uint_as_float(q[j][0][e] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = __uint_as_float(q[j][0][e]);
          v[4 + e] = __uint_as_float(q[j][1][e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float prod = wj[j] * v[e];
        acc[e] = j == 0 ? prod : acc[e] + prod;
      }
    }
    if (residual) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = acc[2 * e] + __uint_as_float(rq[e] << 16);
        acc[2 * e + 1] = acc[2 * e + 1] + __uint_as_float(rq[e] & 0xFFFF0000u);
      }
    }
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = bf16x2_from_float(acc[2 * e], acc[2 * e + 1]);
    *(uint4*)(out + t * H + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

template <bool kBf16, int KMAX>
static void combine_launch(bool g2, dim3 grid, dim3 block, hipStream_t s, const void* y, const int32_t* inv,
                           const float* w, int64_t T, int k, int64_t H, int64_t R, const uint16_t* residual,
                           uint16_t* out) {
  if (g2)
    hipLaunchKernelGGL((combine_kernel<kBf16, KMAX, true>), grid, block, 0, s, y, inv, w, T, k, H, R, residual, out);
  else
    hipLaunchKernelGGL((combine_kernel<kBf16, KMAX, false>), grid, block, 0, s, y, inv, w, T, k, H, R, residual,
                       out);
}

hipError_t launch_combine(const void* y, bool bf16, const int32_t* inv, const float* w, int64_t T, int k,
                          int64_t H, const uint16_t* residual, uint16_t* out, hipStream_t s) {
  const int64_t n = T * (H / 8);
  if (n == 0) return hipSuccess;
  int64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  const int64_t R = T * k;
  // (column blocks of 128 threads, tokens) where T fits the grid's y extent
  const bool g2 = T <= 65535;
  const dim3 grid = g2 ? dim3((unsigned)((H / 8 + 127) / 128), (unsigned)T) : dim3((unsigned)g);
  const dim3 block(g2 ? 128 : 256);
  // slots unrolled up to 8 (top-6 with up to two shared experts) or 16
  if (bf16) {
    if (k <= 8) combine_launch<true, 8>(g2, grid, block, s, y, inv, w, T, k, H, R, residual, out);
    else combine_launch<true, 16>(g2, grid, block, s, y, inv, w, T, k, H, R, residual, out);
  } else {
    if (k <= 8) combine_launch<false, 8>(g2, grid, block, s, y, inv, w, T, k, H, R, residual, out);
    else combine_launch<false, 16>(g2, grid, block, s, y, inv, w, T, k, H, R, residual, out);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
