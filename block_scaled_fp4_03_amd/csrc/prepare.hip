// Weight preparation: a byte permutation of NVFP4 weights into the tiled
// layout the grouped GEMM streams with whole-cache-line loads.
//
// Tiled layout.  The N rows of each group are cut into blocks of 16 rows
// (the last block padded with zero bytes) and K into steps of 256.  Tile
// (g, nb, ks) is 2304 contiguous bytes, tiles ordered by g, then nb, then ks:
//   [0, 1024)     first 16 bytes of each lane:  lane l = r + 16q holds row
//                 nb*16 + r, code bytes ks*128 + 32q + [0, 16)
//   [1024, 2048)  second 16 bytes of each lane: code bytes ks*128 + 32q + [16, 32)
//   [2048, 2304)  scales: lane l holds scale bytes ks*16 + 4q + [0, 4) of row
//                 nb*16 + r
// so a 64-lane wave reads each part with one fully contiguous load, and lane
// (r, q) ends up with the codes and scales of row r for k in
// [ks*256 + 64q, ks*256 + 64q + 64).  Requires K % 256 == 0.
#include "nvfp4_device.hpp"
#include "launch.hpp"

namespace nvfp4 {

// One thread per 4 output bytes.
__global__ __launch_bounds__(256) void prepare_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales, int64_t G, int64_t N,
                                                      int64_t K, uint32_t* __restrict__ out) {
  const int64_t nb_per_g = (N + 15) / 16;
  const int64_t ks_per_row = K / 256;
  const int64_t words = G * nb_per_g * ks_per_row * (kTileBytes / 4);
  const int64_t KB = K / 2, KS = K / 16;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < words;
       w += (int64_t)gridDim.x * blockDim.x) {
    const int64_t tile = w / (kTileBytes / 4);
    const int o = (int)(w - tile * (kTileBytes / 4)) * 4;    // byte offset in the tile
    const int64_t ks = tile % ks_per_row;
    const int64_t gnb = tile / ks_per_row;
    const int64_t nb = gnb % nb_per_g;
    const int64_t g = gnb / nb_per_g;
    int l, b;
    bool is_scale;
    int64_t src_ofs;
    if (o < 2048) {
      const int half = o >= 1024;
      const int oo = o - half * 1024;
      l = oo / 16;
      b = oo % 16;
      is_scale = false;
      src_ofs = ks * 128 + 32 * (l >> 4) + 16 * half + b;
    } else {
      l = (o - 2048) / 4;
      b = 0;
      is_scale = true;
      src_ofs = ks * 16 + 4 * (l >> 4);
    }
    const int64_t row = nb * 16 + (l & 15);
    uint32_t v = 0;
    if (row < N) {
      const uint8_t* src = is_scale ? scales + (g * N + row) * KS + src_ofs : codes + (g * N + row) * KB + src_ofs;
      v = *(const uint32_t*)src;
    }
    out[w] = v;
  }
}

int64_t prepared_bytes(int64_t G, int64_t N, int64_t K) {
  return G * ((N + 15) / 16) * (K / 256) * kTileBytes;
}

hipError_t launch_prepare(const uint8_t* codes, const uint8_t* scales, int64_t G, int64_t N, int64_t K,
                          uint8_t* out, hipStream_t s) {
  const int64_t words = prepared_bytes(G, N, K) / 4;
  if (words == 0) return hipSuccess;
  int64_t grid = (words + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(prepare_kernel, dim3((unsigned)grid), dim3(256), 0, s, codes, scales, G, N, K, (uint32_t*)out);
  return hipGetLastError();
}

}  // namespace nvfp4
