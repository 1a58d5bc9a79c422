// FP8 (E4M3) weight-only projection of the attention output path: bf16
// activations times E4M3 weights with one float32 scale per 128 x 128 block
// (the projection the pages run through an FP8 weight-only einsum: page
// "Current Bug: vLLM produces empty/garbage output", revision e8b289e,
// "Phase 2: CuTeDSL Attention Kernel").
//
//  * fp8_quantize_kernel: one workgroup per 128 x 128 weight block; scale =
//    amax / 448 (1 for an all-zero block), code = sign bit of w plus the E4M3
//    magnitude nearest to |w / scale| (ties to even, saturating).
//  * fp8_gemm_kernel: 128 x 128 output tiles, 4 waves, wave w owns output
//    columns 32 w .. 32 w + 31 and all 128 rows (4 blocks of 32 x 32).  E4M3
//    values convert exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8 with scale
//    1), so every bf16 x E4M3 product of the 32x32x16 bf16 MFMA is exact.  A
//    128-wide k-block has one weight scale per tile (128 output columns are
//    one n-block), so each k-block's sum is formed in its own accumulator and
//    added into the running result as acc += scale * block_sum (one fused
//    multiply-add per value), software-pipelined: the previous block's
//    scaled accumulation and the next weight fragment's conversion run
//    between the current block's MFMAs.  The activations of a k-block go
//    from global memory straight into a swizzled, double-buffered local tile
//    with direct-to-LDS loads, as in the NVFP4 256-row kernel; so do the
//    weights of a k-block (whole 128-byte rows per load, swizzled so that
//    each lane's 64 bytes read back without bank conflicts), each wave
//    copying and reading its own 32 rows.  Row tiles are dealt to the XCDs so
//    that all column tiles of a row tile share one XCD's L2.
#include "nvfp4_device.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t w32x4 __attribute__((ext_vector_type(4)));

constexpr int FB = 128;                 // block edge (scales) = tile edge
constexpr int kFTile = FB * FB * 2;     // bytes of one bf16 activation k-block tile
constexpr int kWTile = FB * FB;         // bytes of one E4M3 weight k-block tile (128 rows x 128 k)

__device__ __forceinline__ int acc_row(int i, int kh) { return 8 * (i >> 2) + 4 * kh + (i & 3); }

}  // namespace

__global__ __launch_bounds__(256) void fp8_quantize_kernel(const float* __restrict__ w, int64_t N, int64_t K,
                                                           int64_t ld_w, uint8_t* __restrict__ codes,
                                                           float* __restrict__ scales) {
  const int64_t nb = blockIdx.y, kb = blockIdx.x;
  const int tid = threadIdx.x;
  const int col = 4 * (tid & 31);          // 4 consecutive k of the block
  const int64_t k = kb * FB + col;
  float v[16][4];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t n = nb * FB + (tid >> 5) + 8 * i;
    if (n < N) {
      const float4 q = *(const float4*)(w + n * ld_w + k);
      v[i][0] = q.x;
      v[i][1] = q.y;
      v[i][2] = q.z;
      v[i][3] = q.w;
    } else {
      v[i][0] = v[i][1] = v[i][2] = v[i][3] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i][e]));
  }
  amax = block_max(amax);
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (tid == 0) scales[nb * (K / FB) + kb] = s;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t n = nb * FB + (tid >> 5) + 8 * i;
    if (n >= N) continue;
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float q = v[i][e] / s;
      const uint32_t c = e4m3_encode(__builtin_fabsf(q)) | ((__float_as_uint(v[i][e]) >> 24) & 0x80u);
      word |= c << (8 * e);
    }
    *(uint32_t*)(codes + n * K + k) = word;
  }
}

__global__ __launch_bounds__(256) void fp8_gemm_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                       int64_t ld_x, const uint8_t* __restrict__ wc,
                                                       const float* __restrict__ ws, int64_t N, void* out,
                                                       int32_t out_bf16, int64_t ld_out, int64_t n_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kFTile + 2 * kWTile];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 31;
  const int kh = lane >> 5;
  // workgroups go to the 8 XCDs round-robin; row tiles are dealt out so
  // that every column tile of a row tile runs on the same XCD (its
  // activation rows then come from that XCD's L2 after the first read,
  // instead of from memory once per column tile)
  const int64_t xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
  const int64_t mt = idx / n_tiles * 8 + xcd;
  const int64_t nt = idx % n_tiles;
  if (mt * FB >= M) return;
  const int64_t m0 = mt * FB, n0 = nt * FB;
  const int64_t nkb = K / FB;

  // activation copies: copy i of wave w fills tile rows 32 w + 4 i .. +3,
  // lane l the physical chunk l % 16 of row 32 w + 4 i + l / 16, which holds
  // logical chunk (l % 16) ^ (row % 16) (k 8 chunk .. 8 chunk + 7 of the
  // k-block); rows past M read row M - 1 (their results are not stored)
  const uint8_t* a_src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 32 * wave + 4 * i + (lane >> 4);
    const int64_t m = m0 + r < M ? m0 + r : M - 1;
    a_src[i] = (const uint8_t*)(x + m * ld_x) + 16 * ((lane & 15) ^ (r & 15));
  }
  auto a_copy = [&](int64_t kb, int buf, int i) {
    __builtin_amdgcn_global_load_lds(
        (const void*)(a_src[i] + kb * 256),
        (__attribute__((address_space(3))) void*)(lds + buf * kFTile + (32 * wave + 4 * i) * 256), 16, 0, 0);
  };
  // weights go through LDS too, so that the loads from memory are whole
  // 128-byte rows: copy i of wave w fills the wave's rows 8 i .. 8 i + 7 of
  // the k-block (lane l: row 8 i + l / 8, physical chunk l % 8 holding
  // logical chunk (l % 8) ^ (row % 8), 16 k each); a wave copies and reads
  // only its own 32 rows.  Lane (c, kh) then reads the 64 bytes
  // [64 kh, 64 kh + 64) of its row c (k-half kh of the block).
  uint8_t* const wlds = lds + 2 * kFTile;
  const uint8_t* w_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * i + (lane >> 3);
    const int64_t nr = n0 + 32 * wave + r < N ? n0 + 32 * wave + r : N - 1;
    w_src[i] = wc + nr * K + 16 * ((lane & 7) ^ (r & 7));
  }
  auto w_copy = [&](int64_t kb, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(
          (const void*)(w_src[i] + kb * FB),
          (__attribute__((address_space(3))) void*)(wlds + buf * kWTile + (32 * wave + 8 * i) * FB), 16, 0, 0);
  };
  auto w_load = [&](int buf, w32x4 (&d)[4]) {
    const uint8_t* row = wlds + buf * kWTile + (32 * wave + c) * FB;
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = *(const w32x4*)(row + 16 * ((4 * kh + q) ^ (c & 7)));
  };
  const float* s_row = ws + (n0 / FB) * nkb;

  // the k-blocks are software-pipelined: while a block's 32 MFMAs run into
  // one set of block accumulators, the previous block's sums (the other
  // set) are scaled into the result 8 values per substep, and the next
  // substep's weight fragment is converted, so that the vector work of a
  // block hides under the matrix work of the next instead of following it
  f32x16 acc[4], tmp_a[4], tmp_b[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    acc[rb] = f32x16{};
    tmp_b[rb] = f32x16{};     // "previous block" of block 0: zeros, scaled by 0
  }
  w32x4 wcur[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) a_copy(0, 0, i);
  w_copy(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  w_load(0, wcur);
  const int x15 = c & 15;
  // weight fragment of substep j (k 16 j .. 16 j + 15 of the block) from the
  // block's loaded words
  auto convert = [&](const w32x4 (&w)[4], int j) {
    const uint32_t w0 = w[j >> 1][2 * (j & 1)], w1 = w[j >> 1][2 * (j & 1) + 1];
    const bf16x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
    const bf16x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
    const bf16x2 b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
    const bf16x2 b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    return bf16x8{b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
  };
  bf16x8 bcur = convert(wcur, 0);
  float s_prev = 0.0f;
  // one k-block: MFMAs into tc, the previous block's tp scaled by s_prev
  auto block = [&](int64_t kb, f32x16 (&tc)[4], const f32x16 (&tp)[4]) {
    const int buf = (int)(kb & 1);
    // the last k-block reloads itself into the unused buffer and registers
    const int64_t kn = kb + 1 < nkb ? kb + 1 : kb;
    w_copy(kn, buf ^ 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) a_copy(kn, buf ^ 1, i);
    const uint8_t* abuf = lds + buf * kFTile + c * 256;
    bf16x8 af[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) af[rb] = *(const bf16x8*)(abuf + rb * 32 * 256 + (((8 * kh) ^ x15) << 4));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bf16x8 bf = bcur;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        tc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[rb], bf, j == 0 ? f32x16{} : tc[rb], 0, 0, 0);
        if (j < 7) af[rb] = *(const bf16x8*)(abuf + rb * 32 * 256 + (((8 * kh + j + 1) ^ x15) << 4));
      }
      if (j < 7) bcur = convert(wcur, j + 1);
      // the previous block: row block j / 2, values 8 (j % 2) .. + 7
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc[j >> 1][8 * (j & 1) + i] = __builtin_fmaf(s_prev, tp[j >> 1][8 * (j & 1) + i], acc[j >> 1][8 * (j & 1) + i]);
      // keep each substep's reads, conversions and updates among its own MFMAs
      __builtin_amdgcn_sched_barrier(0);
    }
    s_prev = s_row[kb];
    __builtin_amdgcn_s_waitcnt(0);     // this wave's copies of the next k-block have landed
    __syncthreads();
    w_load(buf ^ 1, wcur);             // (the wave's own rows: written by its own copies)
    bcur = convert(wcur, 0);
  };
  // two blocks per iteration so that the accumulator sets alternate by name
  int64_t kb = 0;
  for (; kb + 2 <= nkb; kb += 2) {
    block(kb, tmp_a, tmp_b);
    block(kb + 1, tmp_b, tmp_a);
  }
  if (kb < nkb) {
    block(kb, tmp_a, tmp_b);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rb][i] = __builtin_fmaf(s_prev, tmp_a[rb][i], acc[rb][i]);
  } else {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rb][i] = __builtin_fmaf(s_prev, tmp_b[rb][i], acc[rb][i]);
  }

  const int64_t nn = n0 + 32 * wave + c;
  if (nn >= N) return;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t m = m0 + 32 * rb + acc_row(i, kh);
      if (m >= M) continue;
      if (out_bf16)
        ((uint16_t*)out)[m * ld_out + nn] = bf16_from_float(acc[rb][i]);
      else
        ((float*)out)[m * ld_out + nn] = acc[rb][i];
    }
}

hipError_t launch_fp8_quantize(const float* w, int64_t N, int64_t K, int64_t ld_w, uint8_t* codes, float* scales,
                               hipStream_t s) {
  if (N == 0) return hipSuccess;
  hipLaunchKernelGGL(fp8_quantize_kernel, dim3((unsigned)(K / FB), (unsigned)((N + FB - 1) / FB)), dim3(256), 0, s,
                     w, N, K, ld_w, codes, scales);
  return hipGetLastError();
}

hipError_t launch_fp8_gemm(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, const uint8_t* wc, const float* ws,
                           int64_t N, void* out, bool out_bf16, int64_t ld_out, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int64_t n_tiles = (N + FB - 1) / FB;
  const int64_t m_slots = ((M + FB - 1) / FB + 7) / 8 * 8;   // row tiles, padded to the 8 XCDs
  hipLaunchKernelGGL(fp8_gemm_kernel, dim3((unsigned)(m_slots * n_tiles)), dim3(256), 0, s, x, M, K, ld_x, wc, ws, N,
                     out, out_bf16 ? 1 : 0, ld_out, n_tiles);
  return hipGetLastError();
}

}  // namespace nvfp4
