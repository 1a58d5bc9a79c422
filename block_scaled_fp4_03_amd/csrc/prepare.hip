// Weight preparation: a byte permutation of NVFP4 weights into the tiled
// layout the grouped GEMM streams with whole-cache-line loads.
//
// Tiled layout, built around the 32 x 32 x 16 matrix-core instruction
// (lane l = c + 32 kh feeds column c and one of two halves kh of each
// instruction's k range).  The N rows of each group are cut into blocks of
// 32 rows (the last block padded with zero bytes) and K into steps of 256;
// a step is two half-steps h of 128.  Tile (g, nb, ks) is 4608 contiguous
// bytes, tiles ordered by g, then nb, then ks:
//   codes  [h * 2048 + i * 1024 + 16 l, +16), h, i in {0, 1}: row
//          nb * 32 + c, code bytes ks * 128 + 64 h + 32 kh + 16 i + [0, 16)
//   scales [4096 + h * 256 + 4 l, +4): row nb * 32 + c, scale bytes
//          ks * 16 + 8 h + 4 kh + [0, 4)
// so a 64-lane wave reads each part with one fully contiguous load, and in
// half-step h lane (c, kh) holds the 32 code bytes and 4 scales of row c for
// k in [ks * 256 + 128 h + 64 kh, +64).  Requires K % 256 == 0.
#include "nvfp4_device.hpp"
#include "launch.hpp"

namespace nvfp4 {

// One thread per 4 output bytes.
__global__ __launch_bounds__(256) void prepare_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales, int64_t G, int64_t N,
                                                      int64_t K, uint32_t* __restrict__ out) {
  const int64_t nb_per_g = (N + kTileRows - 1) / kTileRows;
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
    int l;
    bool is_scale;
    int64_t src_ofs;
    if (o < 4096) {
      const int h = o >> 11, i = (o >> 10) & 1, oo = o & 1023;
      l = oo >> 4;
      is_scale = false;
      src_ofs = ks * 128 + 64 * h + 32 * (l >> 5) + 16 * i + (oo & 15);
    } else {
      const int h = (o - 4096) >> 8, oo = (o - 4096) & 255;
      l = oo >> 2;
      is_scale = true;
      src_ofs = ks * 16 + 8 * h + 4 * (l >> 5);
    }
    const int64_t row = nb * kTileRows + (l & 31);
    uint32_t v = 0;
    if (row < N) {
      const uint8_t* src = is_scale ? scales + (g * N + row) * KS + src_ofs : codes + (g * N + row) * KB + src_ofs;
      v = *(const uint32_t*)src;
    }
    out[w] = v;
  }
}

int64_t prepared_bytes(int64_t G, int64_t N, int64_t K) {
  return G * ((N + kTileRows - 1) / kTileRows) * (K / 256) * kTileBytes;
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
