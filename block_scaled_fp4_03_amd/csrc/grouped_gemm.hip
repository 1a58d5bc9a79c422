// Grouped GEMM of two NVFP4 operands on the gfx950 matrix cores.
//
//   out[m, n] = alpha(g, n) * sum_k A[m, k] * W[g, n, k]   for m in group g
//
// Both operands arrive as E2M1 codes plus E4M3 block scales.  They are
// dequantised in registers to f16 (exact: e2m1 * e4m3 has at most five
// significant bits and lies in [2^-10, 2688]) and multiplied with
// v_mfma_f32_16x16x32_f16, whose products are exact and whose sums are
// float32.  The per-tensor global scales are applied once, in the epilogue.
//
// MFMA 16x16x32 f16 operand layout (checked on the device): lane l supplies
// row (l % 16) of the 16x32 left operand and column (l % 16) of the 32x16
// right operand, eight consecutive k each, k-slot (l / 16); lane l receives
// D[4 * (l / 16) + i][l % 16], i = 0..3.  Which eight k values a lane feeds is
// our choice as long as both operands make the same choice, which lets every
// lane read long contiguous runs of its own row.
//
// Two kernels:
//  * gemm_rows16 - 16 rows x (4 waves x NBW x 16) columns per workgroup,
//    every wave streaming its own columns over the whole K with no shared
//    memory: the weight-streaming kernel for few rows per group (decode).
//  * gemm_tile   - 128 x 128 tiles, raw codes staged in LDS with double
//    buffering, 2 x 2 waves of 64 x 64: the kernel for many rows per group.
// A workgroup finds its (group, row range) from the device group offsets, so
// the launch needs no host-side knowledge of the group sizes; workgroups past
// the last tile exit at once.
#include "nvfp4_device.hpp"
#include "launch.hpp"

namespace nvfp4 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T clampv(T v, T lo, T hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// The `slot`-th row tile when every group g is cut into ceil(rows_g / BM)
// tiles of BM rows, groups in order.  Executed by a whole wave (all lanes get
// the result).  Offsets are clamped into [0, M] and forced non-decreasing, so
// garbage offsets cannot produce rows outside [0, M).
template <int BM>
__device__ bool find_tile(const int32_t* __restrict__ offsets, int G, int64_t M, int64_t slot, int& g_out,
                          int64_t& r0, int64_t& r1) {
  const int lane = threadIdx.x & 63;
  int64_t base = 0;
  for (int g0 = 0; g0 < G; g0 += 64) {
    const int g = g0 + lane;
    int64_t lo = 0, hi = 0;
    int32_t tiles = 0;
    if (g < G) {
      lo = clampv<int64_t>(offsets[g], 0, M);
      hi = clampv<int64_t>(offsets[g + 1], 0, M);
      if (hi < lo) hi = lo;
      tiles = (int32_t)((hi - lo + BM - 1) / BM);
    }
    int32_t incl = tiles;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    const int32_t excl = incl - tiles;
    const int32_t total = __shfl(incl, 63, 64);
    if (slot < base + total) {
      const bool mine = g < G && slot >= base + excl && slot < base + incl;
      const uint64_t mask = __ballot(mine);
      const int src = __ffsll((unsigned long long)mask) - 1;
      g_out = __shfl(g, src, 64);
      const int32_t lo_s = __shfl((int32_t)lo, src, 64);
      const int32_t hi_s = __shfl((int32_t)hi, src, 64);
      const int32_t ex_s = __shfl(excl, src, 64);
      r0 = lo_s + (slot - base - ex_s) * BM;
      r1 = r0 + BM < hi_s ? r0 + BM : hi_s;
      return true;
    }
    base += total;
  }
  return false;
}

__device__ __forceinline__ float alpha_for(const GemmArgs& p, int g, int64_t n, float a_gs) {
  int s = 0;
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (i < p.n_segs && n >= p.n_seg[i]) s = i;
  return a_gs * p.w_gs[(int64_t)g * p.n_segs + s];
}

__device__ __forceinline__ void store_out(const GemmArgs& p, int64_t m, int64_t n, float v) {
  if (p.out_bf16)
    ((uint16_t*)p.out)[m * p.ld_out + n] = bf16_from_float(v);
  else
    ((float*)p.out)[m * p.ld_out + n] = v;
}

__device__ __forceinline__ uint32_t byte_of(uint32_t w, int i) { return (w >> (8 * i)) & 0xFFu; }

// ---------------------------------------------------------------------------
// gemm_rows16: decode-shaped.  Lane (r = l % 16, q = l / 16).  In the main
// loop a K-step is 256: lane q feeds k in [kb + 64q, kb + 64q + 64), i.e. 32
// contiguous bytes of codes and one 4-byte word of scales of its row, and
// MFMA j (0..7) takes word j of those bytes (block scale byte j / 2).  The
// tail (K % 256) runs K-steps of 32 with lane q feeding [kt + 8q, kt + 8q + 8).
template <int NBW, bool kTiled>
__global__ __launch_bounds__(256) void gemm_rows16(GemmArgs p, int64_t n_tiles) {
  constexpr int BN = 4 * NBW * 16;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int64_t slot = (int64_t)blockIdx.x / n_tiles;
  const int64_t nt = (int64_t)blockIdx.x - slot * n_tiles;
  int g;
  int64_t row0, row1;
  if (!find_tile<16>(p.group_offsets, p.G, p.M, slot, g, row0, row1)) return;
  const int64_t n0 = nt * BN + wave * NBW * 16;
  if (n0 >= p.N) return;
  const int64_t K = p.K;
  const int64_t KB = K / 2;    // code bytes per row
  const int64_t KS = K / 16;   // scale bytes per row

  // A row of this lane
  const int64_t m = row0 + r;
  const bool a_valid = m < row1;
  int64_t a_row = a_valid ? (p.a_row_index ? (int64_t)p.a_row_index[m] : m) : 0;
  a_row = clampv<int64_t>(a_row, 0, p.a_rows > 0 ? p.a_rows - 1 : 0);
  const uint8_t* a_c = p.a_codes + a_row * KB;
  const uint8_t* a_s = p.a_scales + a_row * KS;

  // W rows (output columns) of this lane.  Row-major: the lane's own row.
  // Tiled: the first tile of the lane's 16-row block (the lane offset inside
  // a tile is added at load time); tiles of one block follow each other in k.
  const uint8_t* w_c[NBW];
  const uint8_t* w_s[NBW];
#pragma unroll
  for (int cb = 0; cb < NBW; ++cb) {
    if constexpr (kTiled) {
      const int64_t nb_per_g = (p.N + 15) / 16;
      int64_t nb = (n0 + cb * 16) / 16;
      nb = nb < nb_per_g ? nb : nb_per_g - 1;
      w_c[cb] = p.w_codes + ((int64_t)g * nb_per_g + nb) * (K / 256) * kTileBytes;
      w_s[cb] = w_c[cb];
    } else {
      const int64_t n = clampv<int64_t>(n0 + cb * 16 + r, 0, p.N - 1);
      const int64_t wr = (int64_t)g * p.N + n;
      w_c[cb] = p.w_codes + wr * KB;
      w_s[cb] = p.w_scales + wr * KS;
    }
  }

  floatx4_t acc[NBW];
#pragma unroll
  for (int cb = 0; cb < NBW; ++cb) acc[cb] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // The 256-step loads one 4-byte word of scales per lane, which needs the
  // scale rows (K/16 bytes) to be 4-byte aligned, i.e. K % 64 == 0.
  const int64_t K256 = kTiled ? K : (K % 64 == 0 ? K - K % 256 : 0);
  if (K256 > 0) {
    // software pipeline: the next step's bytes are in flight while the
    // current step is dequantised and multiplied
    u32x4 ac0, ac1, wc0[NBW], wc1[NBW];
    uint32_t as, ws[NBW];
    auto load = [&](int64_t kb, u32x4& c0, u32x4& c1, uint32_t& sc, u32x4 (&d0)[NBW], u32x4 (&d1)[NBW],
                    uint32_t (&sw)[NBW]) {
      const int64_t cofs = kb / 2 + 32 * q;
      const int64_t sofs = kb / 16 + 4 * q;
      if (a_valid) {
        c0 = *(const u32x4*)(a_c + cofs);
        c1 = *(const u32x4*)(a_c + cofs + 16);
        sc = *(const uint32_t*)(a_s + sofs);
      } else {
        c0 = u32x4{0u, 0u, 0u, 0u};
        c1 = c0;
        sc = 0;
      }
#pragma unroll
      for (int cb = 0; cb < NBW; ++cb) {
        if constexpr (kTiled) {
          const uint8_t* t = w_c[cb] + (kb / 256) * kTileBytes;
          d0[cb] = *(const u32x4*)(t + 16 * lane);
          d1[cb] = *(const u32x4*)(t + 1024 + 16 * lane);
          sw[cb] = *(const uint32_t*)(t + 2048 + 4 * lane);
        } else {
          d0[cb] = *(const u32x4*)(w_c[cb] + cofs);
          d1[cb] = *(const u32x4*)(w_c[cb] + cofs + 16);
          sw[cb] = *(const uint32_t*)(w_s[cb] + sofs);
        }
      }
    };
    load(0, ac0, ac1, as, wc0, wc1, ws);
    for (int64_t kb = 0; kb < K256; kb += 256) {
      u32x4 nac0, nac1, nwc0[NBW], nwc1[NBW];
      uint32_t nas, nws[NBW];
      const bool more = kb + 256 < K256;
      if (more) load(kb + 256, nac0, nac1, nas, nwc0, nwc1, nws);
      const uint32_t aw[8] = {ac0.x, ac0.y, ac0.z, ac0.w, ac1.x, ac1.y, ac1.z, ac1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const half8_t af = dequant8(aw[j], scale_pair(byte_of(as, j >> 1)));
#pragma unroll
        for (int cb = 0; cb < NBW; ++cb) {
          const uint32_t ww[8] = {wc0[cb].x, wc0[cb].y, wc0[cb].z, wc0[cb].w,
                                  wc1[cb].x, wc1[cb].y, wc1[cb].z, wc1[cb].w};
          const half8_t bf = dequant8(ww[j], scale_pair(byte_of(ws[cb], j >> 1)));
          acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, acc[cb], 0, 0, 0);
        }
      }
      if (more) {
        ac0 = nac0;
        ac1 = nac1;
        as = nas;
#pragma unroll
        for (int cb = 0; cb < NBW; ++cb) {
          wc0[cb] = nwc0[cb];
          wc1[cb] = nwc1[cb];
          ws[cb] = nws[cb];
        }
      }
    }
  }
  for (int64_t kt = K256; kt < K; kt += 32) {
    const int64_t cofs = kt / 2 + 4 * q;
    const int64_t sofs = (kt + 8 * q) / 16;
    const uint32_t aw = a_valid ? *(const uint32_t*)(a_c + cofs) : 0u;
    const uint32_t asb = a_valid ? (uint32_t)a_s[sofs] : 0u;
    const half8_t af = dequant8(aw, scale_pair(asb));
#pragma unroll
    for (int cb = 0; cb < NBW; ++cb) {
      const uint32_t ww = *(const uint32_t*)(w_c[cb] + cofs);
      const half8_t bf = dequant8(ww, scale_pair((uint32_t)w_s[cb][sofs]));
      acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, acc[cb], 0, 0, 0);
    }
  }

  const float a_gs = *p.a_gs;
#pragma unroll
  for (int cb = 0; cb < NBW; ++cb) {
    const int64_t n = n0 + cb * 16 + r;
    if (n >= p.N) continue;
    const float alpha = alpha_for(p, g, n, a_gs);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t mm = row0 + 4 * q + i;
      if (mm < row1) store_out(p, mm, n, alpha * acc[cb][i]);
    }
  }
}

// ---------------------------------------------------------------------------
// gemm_tile: 128 x 128 output tile per workgroup of 256 threads, K-step 64.
// Per step the raw codes (32 B per row) and scales (4 B per row) of the A and
// W tiles go global -> registers -> LDS (double buffered, one barrier per
// step); each wave then reads its fragments from LDS and dequantises them.
// Lane (r, q) of a 16-row block reads bytes [8q, 8q + 8) of its row, i.e. k in
// [16q, 16q + 16) of the step, one scale block; MFMA substep s (0, 1) takes
// word s of those bytes.
constexpr int TBM = 128, TBN = 128, TBK = 64;

template <bool kTiled>
__global__ __launch_bounds__(256) void gemm_tile(GemmArgs p, int64_t n_tiles) {
  __shared__ uint8_t lds_ac[2][TBM * 32];
  __shared__ uint8_t lds_wc[2][TBN * 32];
  __shared__ uint32_t lds_as[2][TBM];
  __shared__ uint32_t lds_ws[2][TBN];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int64_t slot = (int64_t)blockIdx.x / n_tiles;
  const int64_t nt = (int64_t)blockIdx.x - slot * n_tiles;
  int g;
  int64_t row0, row1;
  if (!find_tile<TBM>(p.group_offsets, p.G, p.M, slot, g, row0, row1)) return;
  const int64_t n0 = nt * TBN;
  const int64_t K = p.K;
  const int64_t KB = K / 2;
  const int64_t KS = K / 16;

  // global -> LDS copy assignment: codes, thread t moves 16 B of row t / 2;
  // scales, threads 0..127 move the A word of row t, 128..255 the W word.
  const int crow = tid >> 1;
  const int chalf = tid & 1;
  int64_t am = row0 + crow;
  const bool a_ok = am < row1;
  int64_t a_row = a_ok ? (p.a_row_index ? (int64_t)p.a_row_index[am] : am) : 0;
  a_row = clampv<int64_t>(a_row, 0, p.a_rows > 0 ? p.a_rows - 1 : 0);
  const uint8_t* a_c = p.a_codes + a_row * KB + 16 * chalf;
  // W codes: row-major, thread t moves 16 B of row t / 2 like A.  Tiled,
  // thread t takes 16-row block t / 32, half (t / 16) % 2, row t % 16: the
  // k-step of 64 is one quarter (q' = ks % 4) of a 256-k tile, whose halves
  // sit at 256 q' + 16 r and 1024 + 256 q' + 16 r.
  const int w_lds_row = kTiled ? ((tid >> 5) * 16 + (tid & 15)) : crow;
  const int w_half = kTiled ? ((tid >> 4) & 1) : chalf;
  const int64_t nb_per_g = (p.N + 15) / 16;
  const uint8_t* w_c;
  if constexpr (kTiled) {
    int64_t nb = n0 / 16 + (tid >> 5);
    nb = nb < nb_per_g ? nb : nb_per_g - 1;
    w_c = p.w_codes + ((int64_t)g * nb_per_g + nb) * (K / 256) * kTileBytes + 1024 * w_half + 16 * (tid & 15);
  } else {
    const int64_t wn_row = (int64_t)g * p.N + clampv<int64_t>(n0 + crow, 0, p.N - 1);
    w_c = p.w_codes + wn_row * KB + 16 * chalf;
  }
  const int srow = tid & 127;
  const uint8_t* s_src;
  if (tid < 128) {
    int64_t sm = row0 + srow;
    int64_t sr = sm < row1 ? (p.a_row_index ? (int64_t)p.a_row_index[sm] : sm) : 0;
    sr = clampv<int64_t>(sr, 0, p.a_rows > 0 ? p.a_rows - 1 : 0);
    s_src = p.a_scales + sr * KS;
  } else if constexpr (kTiled) {
    int64_t nb = n0 / 16 + (srow >> 4);
    nb = nb < nb_per_g ? nb : nb_per_g - 1;
    s_src = p.w_codes + ((int64_t)g * nb_per_g + nb) * (K / 256) * kTileBytes + 2048 + 4 * (srow & 15);
  } else {
    s_src = p.w_scales + ((int64_t)g * p.N + clampv<int64_t>(n0 + srow, 0, p.N - 1)) * KS;
  }

  floatx4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t nk = K / TBK;
  u32x4 ra, rw;
  uint32_t rs;
  auto gload = [&](int64_t ks) {
    ra = *(const u32x4*)(a_c + ks * 32);
    if constexpr (kTiled) {
      const int64_t tofs = (ks >> 2) * kTileBytes + 256 * (ks & 3);
      rw = *(const u32x4*)(w_c + tofs);
      rs = tid < 128 ? *(const uint32_t*)(s_src + ks * 4)
                     : *(const uint32_t*)(s_src + (ks >> 2) * kTileBytes + 64 * (ks & 3));
    } else {
      rw = *(const u32x4*)(w_c + ks * 32);
      rs = *(const uint32_t*)(s_src + ks * 4);
    }
  };
  auto lstore = [&](int buf) {
    *(u32x4*)(&lds_ac[buf][crow * 32 + 16 * chalf]) = ra;
    *(u32x4*)(&lds_wc[buf][w_lds_row * 32 + 16 * w_half]) = rw;
    if (tid < 128) lds_as[buf][srow] = rs;
    else lds_ws[buf][srow] = rs;
  };
  gload(0);
  lstore(0);
  __syncthreads();
  for (int64_t ks = 0; ks < nk; ++ks) {
    const int buf = (int)(ks & 1);
    const bool more = ks + 1 < nk;
    if (more) gload(ks + 1);
    // fragments of this wave: 4 row blocks of A, 4 column blocks of W
    uint2 af_raw[4], bf_raw[4];
    uint32_t af_s[4], bf_s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ar = wm * 64 + i * 16 + r;
      af_raw[i] = *(const uint2*)(&lds_ac[buf][ar * 32 + 8 * q]);
      af_s[i] = byte_of(lds_as[buf][ar], q);
      const int br = wn * 64 + i * 16 + r;
      bf_raw[i] = *(const uint2*)(&lds_wc[buf][br * 32 + 8 * q]);
      bf_s[i] = byte_of(lds_ws[buf][br], q);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      half8_t bfr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[j] = dequant8(s ? bf_raw[j].y : bf_raw[j].x, scale_pair(bf_s[j]));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const half8_t afr = dequant8(s ? af_raw[i].y : af_raw[i].x, scale_pair(af_s[i]));
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr, bfr[j], acc[i][j], 0, 0, 0);
      }
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
  }

  const float a_gs = *p.a_gs;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + wn * 64 + j * 16 + r;
    if (n >= p.N) continue;
    const float alpha = alpha_for(p, g, n, a_gs);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t mm = row0 + wm * 64 + i * 16 + 4 * q + e;
        if (mm < row1) store_out(p, mm, n, alpha * acc[i][j][e]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  const bool many_rows = a.M >= (int64_t)64 * a.G && a.K % TBK == 0;
  if (many_rows) {
    const int64_t n_tiles = (a.N + TBN - 1) / TBN;
    const int64_t slots = (a.M + TBM - 1) / TBM + a.G;
    if (a.w_tiled)
      hipLaunchKernelGGL(gemm_tile<true>, dim3((unsigned)(slots * n_tiles)), dim3(256), 0, s, a, n_tiles);
    else
      hipLaunchKernelGGL(gemm_tile<false>, dim3((unsigned)(slots * n_tiles)), dim3(256), 0, s, a, n_tiles);
  } else {
    constexpr int NBW = 4;
    const int64_t n_tiles = (a.N + 4 * NBW * 16 - 1) / (4 * NBW * 16);
    const int64_t slots = (a.M + 15) / 16 + a.G;
    if (a.w_tiled)
      hipLaunchKernelGGL((gemm_rows16<NBW, true>), dim3((unsigned)(slots * n_tiles)), dim3(256), 0, s, a, n_tiles);
    else
      hipLaunchKernelGGL((gemm_rows16<NBW, false>), dim3((unsigned)(slots * n_tiles)), dim3(256), 0, s, a,
                         n_tiles);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
