// Internal interface between the C ABI layer (capi.cpp) and the kernel
// translation units: small device reductions shared by several kernels, and
// the host-side launchers each .hip file defines.  Launchers assume their
// arguments were validated by the C ABI layer and only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

#ifdef __HIPCC__
// Max over a wave64, every lane gets the result.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Max over a block of at most 1024 threads (a multiple of 64); every thread
// gets the result.  Uses 64 bytes of shared memory.
__device__ __forceinline__ float block_max(float v) {
  __shared__ float part[16];
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) part[w] = v;
  __syncthreads();
  const int nw = (blockDim.x + 63) >> 6;
  float r = 0.0f;
  for (int i = 0; i < nw; ++i) r = __builtin_fmaxf(r, part[i]);
  __syncthreads();
  return r;
}

// gs = amax / (6 * 448) in the dequantisation direction; 1.0 for amax == 0.
__device__ __forceinline__ float global_scale_from_amax(float amax) {
  return amax == 0.0f ? 1.0f : amax / 2688.0f;
}
#endif

// One tile of the prepared (tiled) weight layout: 32 rows x 256 k, codes
// (4096 B) then scales (512 B).
constexpr int kTileRows = 32;
constexpr int kTileBytes = 4608;
// Largest K of the tiled layout: one 32-row block's K range (K / 256 tiles)
// stays far below 2^31 bytes, the reach of the kernels' buffer resources.
constexpr int64_t kMaxTiledK = (int64_t)1 << 24;

// --- launchers (defined in the .hip files) --------------------------------
hipError_t launch_quantize(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld_x,
                           const float* gs, uint8_t* codes, uint8_t* scales, uint16_t* dq, hipStream_t s);
int64_t amax_chunks(int64_t n);
// The no-allocation entry point's scratch: floats per device, and its device
// address on the current device (looked up once per device).
constexpr int64_t kNoAllocScratchFloats = 65536;
hipError_t noalloc_scratch(float** ptr);
hipError_t launch_global_scale(const void* x, bool bf16, int64_t batch, int64_t n, int64_t stride,
                               float* gs_out, float* partial, hipStream_t s);

hipError_t launch_route_permute(const float* logits, int64_t T, int E, int k, int ns, int32_t* ids,
                                float* w, int32_t* offsets, int32_t* sorted_ids, int32_t* inv, hipStream_t s);

int64_t prepared_bytes(int64_t G, int64_t N, int64_t K);
hipError_t launch_prepare(const uint8_t* codes, const uint8_t* scales, int64_t G, int64_t N, int64_t K,
                          uint8_t* out, hipStream_t s);

struct GemmArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_gs;
  int64_t a_rows;
  const int32_t* a_row_index;  // nullable
  const uint16_t* a_dq;        // nullable: f16 [a_rows, K], e2m1 * e4m3 of A
  const uint8_t* w_codes;      // row-major codes, or the tiled buffer
  const uint8_t* w_scales;     // row-major scales (unused when tiled)
  int32_t w_tiled;             // 1: w_codes is the prepared tiled layout
  const float* w_gs;
  int32_t n_seg[5];            // n_seg[0..n_segs], padded with N
  int32_t n_segs;
  const int32_t* group_offsets;
  int32_t G;
  int64_t M, N, K;
  void* out;
  int32_t out_bf16;
  int64_t ld_out;
  // fused SiLU-requant epilogue (fuse = 1, tiled weights): N = 2 I with the
  // gate in columns [0, I) and the up projection in [I, 2 I); instead of
  // `out`, h = SiLU(gate) * up is written re-quantised with h_gs
  int32_t fuse;
  const float* h_gs;
  uint8_t* h_codes;    // [M, I/2]
  uint8_t* h_scales;   // [M, I/16]
  uint16_t* h_dq;      // nullable: [M, I] f16, e2m1 * e4m3 of h
  // fuse = 1 with h_f32: h is written in float32 instead ([M, I], row pitch
  // I; h_gs, h_codes, h_scales and h_dq unused), and each wave of the launch
  // stores the largest |h| of its rows at h_amax[4 * workgroup + wave] (the
  // launcher zeroes the h_amax_n entries first)
  float* h_f32;
  float* h_amax;
  int64_t h_amax_n;
  // split-K (splits > 1): raw partial sums [splits, M, N] float32 in ws,
  // added in split order and scaled by alpha by a second kernel
  int32_t splits;
  float* ws;
};
// split-K factor the launcher uses for these sizes (1: none) and the bytes
// of partial sums it needs
int32_t gemm_splitk_splits(int64_t G, int64_t M, int64_t N, int64_t K, bool tiled);
size_t gemm_splitk_bytes(int64_t G, int64_t M, int64_t N, int64_t K, bool tiled);
// true when launch_grouped_gemm runs the matrix-core tiles (which read a_dq)
bool gemm_uses_big_tiles(int64_t G, int64_t M, int64_t K, bool tiled);
// true when launch_tiled, given A in f16 form and a split-K workspace, runs
// one group of at most 128 rows on the 128-row tiles split over K
bool gemm_small_split(int64_t G, int64_t M, bool tiled);
hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t s);
// entries of h_amax that a fused launch with h_f32 of these sizes may write
// (four per workgroup of the largest grid it can use)
int64_t gemm_silu_f32_amax_slots(int64_t G, int64_t M, int64_t I);
// the expert MLP in one persistent launch: l1 the first GEMM with the fused
// SiLU-requant epilogue, l2 the second GEMM over the same groups (A = h);
// ctr holds moe_persistent_counters(G, M) int32 counters
int64_t moe_persistent_counters(int64_t G, int64_t M);
hipError_t launch_moe_persistent(const GemmArgs& l1, const GemmArgs& l2, int32_t* ctr, int32_t spin_limit,
                                 hipStream_t s);

hipError_t launch_fp8_quantize(const float* w, int64_t N, int64_t K, int64_t ld_w, uint8_t* codes, float* scales,
                               hipStream_t s);
hipError_t launch_fp8_gemm(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, const uint8_t* wc, const float* ws,
                           int64_t N, void* out, bool out_bf16, int64_t ld_out, hipStream_t s);

hipError_t launch_silu_mul_requant(const void* gu, bool bf16, int64_t M, int64_t I, int64_t ld,
                                   const float* gs_h, uint8_t* codes, uint8_t* scales, uint16_t* dq,
                                   hipStream_t s);
int64_t silu_amax_chunks(int64_t M, int64_t I);
hipError_t launch_silu_mul_global_scale(const void* gu, bool bf16, int64_t M, int64_t I, int64_t ld,
                                        float* gs_out, float* partial, hipStream_t s);

hipError_t launch_read_probe(const void* buf, int64_t bytes, void* sink, hipStream_t s);
hipError_t launch_mfma_probe(int64_t iters, int64_t workgroups, void* sink, hipStream_t s);

hipError_t launch_combine(const void* y, bool bf16, const int32_t* inv, const float* w, int64_t T,
                          int k, int64_t H, const uint16_t* residual, uint16_t* out, hipStream_t s);

}  // namespace nvfp4
