// Grouped GEMM of two NVFP4 operands on the gfx950 matrix cores.
//
//   out[m, n] = alpha(g, n) * sum_k A[m, k] * W[g, n, k]   for m in group g
//
// Both operands arrive as E2M1 codes plus E4M3 block scales.  They are
// dequantised in registers to f16 (exact: e2m1 * e4m3 has at most five
// significant bits and lies in [2^-10, 2688]) and multiplied on the matrix
// cores, whose products are exact and whose sums are float32.  The
// per-tensor global scales are applied once, in the epilogue.
//
// Matrix-core instructions (lane layouts checked on the device):
//  * v_mfma_f32_32x32x16_f16: lane l = c + 32 kh supplies row c of the 32x16
//    left operand and column c of the 16x32 right operand, eight k each (k
//    half kh); lane l receives D[8 (i / 4) + 4 kh + (i % 4)][c], i = 0..15.
//    On gfx950 it sustains ~1.9 PFLOP/s, twice the 16x16x32 form, so the
//    kernels over prepared (tiled) weights use it.
//  * v_mfma_f32_16x16x32_f16: lane l = r + 16 q supplies row/column r, eight
//    k each (k slot q); lane l receives D[4 q + i][r].  Used by the fallback
//    kernels over row-major weights.
// Which k values a lane feeds is our choice as long as both operands make
// the same choice, which lets every lane read long contiguous runs.
//
// Kernels:
//  * gemm_stream32 - prepared weights, 32*RB rows x (4 waves x NBW x 32)
//    columns per workgroup, every wave streaming its columns of W over the
//    whole K with no shared memory: the weight-streaming kernel for few rows
//    per group (decode) and for the rows a 256-row tile leaves over when A
//    comes without its f16 form.
//  * gemm_big32_dq4 / gemm_dq4_split - prepared weights and A in f16 form,
//    128 x 256 tiles (the last tile of a group 32, 64 or 128 rows high), A
//    copied into LDS by DMA, two workgroups per compute unit: many rows per
//    group (prefill), and one group split over K.
//  * gemm_big32    - prepared weights, A as codes only, 256 x 256 tiles, A
//    dequantised once per workgroup into LDS (fallback).
//  * gemm_stream16 / gemm_tile16 - row-major weights (any K % 32 == 0).
//  * splitk_reduce4 / splitk_reduce / splitk_reduce_silu_requant - the
//    split-K partial sums added in range order, times alpha, to the output
//    or (the first GEMM of the expert MLP) through SiLU-requant.
// A workgroup finds its (group, row range) from the device group offsets, so
// the launch needs no host-side knowledge of the group sizes; workgroups past
// the last tile exit at once.
#include <algorithm>

#include "nvfp4_device.hpp"
#include "launch.hpp"

namespace nvfp4 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T clampv(T v, T lo, T hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// Inclusive prefix sum over the 64 lanes of a wave in six DPP adds: shifts by
// 1, 2, 4 and 8 lanes within each row of 16 (lanes shifted in from outside the
// row add 0), then the last lane of row 0 (of row 2) is added to row 1 (row 3),
// and lane 31 to rows 2 and 3.  No local-memory round trips, unlike a
// shuffle-based scan.
// x of another lane of the same DPP row (16 lanes), by a DPP control that
// reads within the row (every lane has a source)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ int32_t wave_incl_scan(int32_t x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2 and 3
  return x;
}

// The `slot`-th row tile of a launch.  Every group g (rows [lo, hi) from the
// device offsets) contributes the rows [start, hi): start = lo, or, when
// skip_bm > 0, the rows another launch leaves over, which tiles skip_bm rows
// at a time and takes the last partial tile too if it has at least skip_min
// rows.  They are cut into tiles of bm rows; a last partial tile is kept if
// it has at least last_min rows (1: always, bm: never).  Groups are taken in
// order.  Executed by a whole wave (all lanes get the result).  Offsets are
// clamped into [0, M] and forced non-decreasing, so garbage offsets cannot
// produce rows outside [0, M).
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int G, int64_t M, int64_t slot, int bm,
                                          int last_min, int skip_bm, int skip_min, int& g_out, int64_t& r0,
                                          int64_t& r1) {
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
      if (skip_bm > 0) {
        const int64_t rest = (hi - lo) % skip_bm;
        lo = rest >= skip_min ? hi : hi - rest;
      }
      tiles = (int32_t)((hi - lo) / bm + ((hi - lo) % bm >= last_min ? 1 : 0));
    }
    const int32_t incl = wave_incl_scan(tiles);
    const int32_t excl = incl - tiles;
    const int32_t total = __builtin_amdgcn_readlane(incl, 63);
    if (slot < base + total) {
      const bool mine = g < G && slot >= base + excl && slot < base + incl;
      const uint64_t mask = __ballot(mine);
      if (mask == 0) return false;   // (cannot happen: some lane's range holds the slot)
      const int src = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)mask) - 1);
      g_out = __builtin_amdgcn_readlane(g, src);
      const int32_t lo_s = __builtin_amdgcn_readlane((int32_t)lo, src);
      const int32_t hi_s = __builtin_amdgcn_readlane((int32_t)hi, src);
      const int32_t ex_s = __builtin_amdgcn_readlane(excl, src);
      r0 = lo_s + (slot - base - ex_s) * bm;
      r1 = r0 + bm < hi_s ? r0 + bm : hi_s;
      return r0 < r1;
    }
    base += total;
  }
  return false;
}

// find_tile with every offset loaded before the scan (one memory round trip
// instead of one per 64 groups), for kernels with registers to spare at the
// start of a tile.
constexpr int kMaxChunks = 16;   // groups in chunks of 64, up to 1024 groups
constexpr int kMaxGroups = 64 * kMaxChunks;

__device__ __forceinline__ bool find_tile_batched(const int32_t* __restrict__ offsets, int G, int64_t M, int64_t slot, int bm,
                                          int last_min, int skip_bm, int skip_min, int& g_out, int64_t& r0,
                                          int64_t& r1) {
  const int lane = threadIdx.x & 63;
  // all the offsets first (one memory round trip), then the scan
  int32_t lo_c[kMaxChunks], hi_c[kMaxChunks];
#pragma unroll
  for (int ch = 0; ch < kMaxChunks; ++ch) {
    const int g = ch * 64 + lane;
    lo_c[ch] = 0;
    hi_c[ch] = 0;
    if (ch * 64 < G && g < G) {
      lo_c[ch] = offsets[g];
      hi_c[ch] = offsets[g + 1];
    }
  }
  int64_t base = 0;
#pragma unroll
  for (int ch = 0; ch < kMaxChunks; ++ch) {
    if (ch * 64 >= G) break;
    const int g = ch * 64 + lane;
    int64_t lo = 0, hi = 0;
    int32_t tiles = 0;
    if (g < G) {
      lo = clampv<int64_t>(lo_c[ch], 0, M);
      hi = clampv<int64_t>(hi_c[ch], 0, M);
      if (hi < lo) hi = lo;
      if (skip_bm > 0) {
        const int64_t rest = (hi - lo) % skip_bm;
        lo = rest >= skip_min ? hi : hi - rest;
      }
      tiles = (int32_t)((hi - lo) / bm + ((hi - lo) % bm >= last_min ? 1 : 0));
    }
    const int32_t incl = wave_incl_scan(tiles);
    const int32_t excl = incl - tiles;
    const int32_t total = __builtin_amdgcn_readlane(incl, 63);
    if (slot < base + total) {
      const bool mine = g < G && slot >= base + excl && slot < base + incl;
      const uint64_t mask = __ballot(mine);
      if (mask == 0) return false;   // (cannot happen: some lane's range holds the slot)
      const int src = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)mask) - 1);
      g_out = __builtin_amdgcn_readlane(g, src);
      const int32_t lo_s = __builtin_amdgcn_readlane((int32_t)lo, src);
      const int32_t hi_s = __builtin_amdgcn_readlane((int32_t)hi, src);
      const int32_t ex_s = __builtin_amdgcn_readlane(excl, src);
      r0 = lo_s + (slot - base - ex_s) * bm;
      r1 = r0 + bm < hi_s ? r0 + bm : hi_s;
      return r0 < r1;
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
// gemm_stream16: the weight-streaming kernel over row-major weights
// (16x16x32 instruction).  A workgroup computes 16*RB rows x (4 waves x NBW x
// 16) columns; every wave streams its NBW 16-column blocks of W over the
// whole K with no shared memory and no barriers, one K-step prefetched
// ahead.  Lane (r = l % 16, q = l / 16).  A K-step is 256: lane q
// feeds k in [kb + 64q, kb + 64q + 64), i.e. 32 contiguous bytes of codes and
// one 4-byte word of scales of its row, and MFMA j (0..7) takes word j of
// those bytes (block scale byte j / 2).  The tail (K % 256) runs K-steps of
// 32 with lane q feeding [kt + 8q, kt + 8q + 8).
template <int NBW, int RB>
__global__ __launch_bounds__(256) void gemm_stream16(GemmArgs p, int64_t n_tiles, int skip_bm) {
  constexpr int BN = 4 * NBW * 16;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int64_t slot = (int64_t)blockIdx.x / n_tiles;
  const int64_t nt = (int64_t)blockIdx.x - slot * n_tiles;
  int g;
  int64_t row0, row1;
  if (!find_tile(p.group_offsets, p.G, p.M, slot, 16 * RB, 1, skip_bm, skip_bm, g, row0, row1)) return;
  const int64_t n0 = nt * BN + wave * NBW * 16;
  if (n0 >= p.N) return;
  const int64_t K = p.K;
  const int64_t KB = K / 2;    // code bytes per row
  const int64_t KS = K / 16;   // scale bytes per row

  // A rows of this lane: row0 + 16 rb + r
  bool a_valid[RB];
  const uint8_t* a_c[RB];
  const uint8_t* a_s[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t m = row0 + 16 * rb + r;
    a_valid[rb] = m < row1;
    int64_t a_row = a_valid[rb] ? (p.a_row_index ? (int64_t)p.a_row_index[m] : m) : 0;
    a_row = clampv<int64_t>(a_row, 0, p.a_rows > 0 ? p.a_rows - 1 : 0);
    a_c[rb] = p.a_codes + a_row * KB;
    a_s[rb] = p.a_scales + a_row * KS;
  }

  // W rows (output columns) of this lane
  const uint8_t* w_c[NBW];
  const uint8_t* w_s[NBW];
#pragma unroll
  for (int cb = 0; cb < NBW; ++cb) {
    const int64_t n = clampv<int64_t>(n0 + cb * 16 + r, 0, p.N - 1);
    const int64_t wr = (int64_t)g * p.N + n;
    w_c[cb] = p.w_codes + wr * KB;
    w_s[cb] = p.w_scales + wr * KS;
  }

  floatx4_t acc[RB][NBW];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < NBW; ++cb) acc[rb][cb] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // The 256-step loads one 4-byte word of scales per lane, which needs the
  // scale rows (K/16 bytes) to be 4-byte aligned, i.e. K % 64 == 0.
  const int64_t K256 = K % 64 == 0 ? K - K % 256 : 0;
  if (K256 > 0) {
    // software pipeline: the next step's bytes are in flight while the
    // current step is dequantised and multiplied
    u32x4 ac0[RB], ac1[RB], wc0[NBW], wc1[NBW];
    uint32_t as[RB], ws[NBW];
    auto load = [&](int64_t kb, u32x4 (&c0)[RB], u32x4 (&c1)[RB], uint32_t (&sc)[RB], u32x4 (&d0)[NBW],
                    u32x4 (&d1)[NBW], uint32_t (&sw)[NBW]) {
      const int64_t cofs = kb / 2 + 32 * q;
      const int64_t sofs = kb / 16 + 4 * q;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (a_valid[rb]) {
          c0[rb] = *(const u32x4*)(a_c[rb] + cofs);
          c1[rb] = *(const u32x4*)(a_c[rb] + cofs + 16);
          sc[rb] = *(const uint32_t*)(a_s[rb] + sofs);
        } else {
          c0[rb] = u32x4{0u, 0u, 0u, 0u};
          c1[rb] = c0[rb];
          sc[rb] = 0;
        }
      }
#pragma unroll
      for (int cb = 0; cb < NBW; ++cb) {
        d0[cb] = *(const u32x4*)(w_c[cb] + cofs);
        d1[cb] = *(const u32x4*)(w_c[cb] + cofs + 16);
        sw[cb] = *(const uint32_t*)(w_s[cb] + sofs);
      }
    };
    load(0, ac0, ac1, as, wc0, wc1, ws);
    for (int64_t kb = 0; kb < K256; kb += 256) {
      u32x4 nac0[RB], nac1[RB], nwc0[NBW], nwc1[NBW];
      uint32_t nas[RB], nws[NBW];
      const bool more = kb + 256 < K256;
      if (more) load(kb + 256, nac0, nac1, nas, nwc0, nwc1, nws);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        half8_t bf[NBW];
#pragma unroll
        for (int cb = 0; cb < NBW; ++cb) {
          const uint32_t w = j < 4 ? wc0[cb][j] : wc1[cb][j - 4];
          bf[cb] = dequant8(w, scale_pair(byte_of(ws[cb], j >> 1)));
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const uint32_t aw = j < 4 ? ac0[rb][j] : ac1[rb][j - 4];
          const half8_t af = dequant8(aw, scale_pair(byte_of(as[rb], j >> 1)));
#pragma unroll
          for (int cb = 0; cb < NBW; ++cb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[cb], acc[rb][cb], 0, 0, 0);
        }
      }
      if (more) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          ac0[rb] = nac0[rb];
          ac1[rb] = nac1[rb];
          as[rb] = nas[rb];
        }
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
    half8_t bf[NBW];
#pragma unroll
    for (int cb = 0; cb < NBW; ++cb) {
      const uint32_t ww = *(const uint32_t*)(w_c[cb] + cofs);
      bf[cb] = dequant8(ww, scale_pair((uint32_t)w_s[cb][sofs]));
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const uint32_t aw = a_valid[rb] ? *(const uint32_t*)(a_c[rb] + cofs) : 0u;
      const uint32_t asb = a_valid[rb] ? (uint32_t)a_s[rb][sofs] : 0u;
      const half8_t af = dequant8(aw, scale_pair(asb));
#pragma unroll
      for (int cb = 0; cb < NBW; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[cb], acc[rb][cb], 0, 0, 0);
    }
  }

  const float a_gs = *p.a_gs;
#pragma unroll
  for (int cb = 0; cb < NBW; ++cb) {
    const int64_t n = n0 + cb * 16 + r;
    if (n >= p.N) continue;
    const float alpha = alpha_for(p, g, n, a_gs);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t mm = row0 + 16 * rb + 4 * q + i;
        if (mm < row1) store_out(p, mm, n, alpha * acc[rb][cb][i]);
      }
  }
}

// ---------------------------------------------------------------------------
// gemm_tile16: 128 x 128 output tile per workgroup (row-major weights) of 256 threads, K-step 64.
// Per step the raw codes (32 B per row) and scales (4 B per row) of the A and
// W tiles go global -> registers -> LDS (double buffered, one barrier per
// step); each wave then reads its fragments from LDS and dequantises them.
// Lane (r, q) of a 16-row block reads bytes [8q, 8q + 8) of its row, i.e. k in
// [16q, 16q + 16) of the step, one scale block; MFMA substep s (0, 1) takes
// word s of those bytes.
constexpr int TBM = 128, TBN = 128, TBK = 64;

__global__ __launch_bounds__(256) void gemm_tile16(GemmArgs p, int64_t n_tiles) {
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
  if (!find_tile(p.group_offsets, p.G, p.M, slot, TBM, 1, 0, 0, g, row0, row1)) return;
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
  // W codes: thread t moves 16 B of row t / 2 like A
  const int64_t wn_row = (int64_t)g * p.N + clampv<int64_t>(n0 + crow, 0, p.N - 1);
  const uint8_t* w_c = p.w_codes + wn_row * KB + 16 * chalf;
  const int srow = tid & 127;
  const uint8_t* s_src;
  if (tid < 128) {
    int64_t sm = row0 + srow;
    int64_t sr = sm < row1 ? (p.a_row_index ? (int64_t)p.a_row_index[sm] : sm) : 0;
    sr = clampv<int64_t>(sr, 0, p.a_rows > 0 ? p.a_rows - 1 : 0);
    s_src = p.a_scales + sr * KS;
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
    rw = *(const u32x4*)(w_c + ks * 32);
    rs = *(const uint32_t*)(s_src + ks * 4);
  };
  auto lstore = [&](int buf) {
    *(u32x4*)(&lds_ac[buf][crow * 32 + 16 * chalf]) = ra;
    *(u32x4*)(&lds_wc[buf][crow * 32 + 16 * chalf]) = rw;
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
// Kernels over prepared (tiled) weights, 32x32x16 instruction.  In half-step
// h of K-step ks, lane l = c + 32 kh feeds k in [ks*256 + 128h + 64kh, +64):
// substep j (0..7) takes k [.. + 8j, +8), i.e. code word j of the lane's 32
// bytes and scale byte j / 2 of its scale word, for A and W alike.

typedef float floatx16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ floatx16_t mfma32(half8_t a, half8_t b, floatx16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Row of D held in accumulator element i by a lane of k half kh.
__device__ __forceinline__ int acc32_row(int i, int kh) { return 8 * (i >> 2) + 4 * kh + (i & 3); }

// Fused epilogue of the first GEMM: the wave holds gate column block j in
// acc[rb][0] and up column block I/32 + j in acc[rb][1] (32x32 accumulator
// layout: lane l = c + 32 kh has column c, rows 32 rb + acc32_row(i, kh)).
// Each value is formed exactly as the unfused GEMM stores it (alpha times
// the sum, float32), then h = SiLU(gate) * up and its NVFP4 re-quantisation
// follow the operation sequence of silu_mul_requant, so codes, scales and
// the f16 copy are identical to the unfused pair of launches.
// h of a 32-row block goes through the wave's own staging area in local
// memory (32 rows x kHStride floats, st) and comes back one quantisation
// block per lane: lane l takes row l % 32, columns 32 j + 16 (l / 32) .. +15,
// so the block's amax, scale, 16 codes and f16 copy are formed once, by one
// lane, and stored as 8 + 1 + 32 contiguous bytes.
constexpr int kHStride = 36;   // floats per staged row: 32, plus 4 to shift the next row's banks
template <int RB>
__device__ __forceinline__ void silu_requant_epilogue(const GemmArgs& p, const floatx16_t (&acc)[RB][2], int g,
                                                      int64_t row0, int64_t row1, int64_t j, int lane, float* st) {
  const int c = lane & 31;
  const int kh = lane >> 5;
  const int64_t I = p.N / 2;
  if (32 * j >= I) return;  // uniform in the wave
  const float a_gs = *p.a_gs;
  const float alpha_g = a_gs * p.w_gs[(int64_t)g * 2];
  const float alpha_u = a_gs * p.w_gs[(int64_t)g * 2 + 1];
  const bool to_f32 = p.h_f32 != nullptr;
  const float gs = to_f32 ? 0.0f : *p.h_gs;
  const int r = lane & 31, hb = lane >> 5;      // after the transpose: row r, half hb of the 32 columns
  const int64_t hcol = 32 * j + 16 * hb;
  float wmax = 0.0f;     // float32 h: the largest |h| of this wave's rows
  const int64_t rows = row1 - row0;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // elements 4q .. 4q + 3 hold rows 32 rb + 8q .. + 7 (both lane
      // halves): skipped, uniformly, where all of them lie past the tile's
      // last row (their staged values are then stale, and only rows past
      // the last read them back, whose results are never stored)
      if (32 * rb + 8 * (i >> 2) >= rows) continue;
      const float gv = alpha_g * acc[rb][0][i];
      const float uv = alpha_u * acc[rb][1][i];
      st[acc32_row(i, kh) * kHStride + c] = silu_mul(gv, uv);
    }
    // one wave's local-memory operations complete in issue order: the reads
    // below see the writes above, and the next block's writes follow them
    float h[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const floatx4_t v = *(const floatx4_t*)(st + r * kHStride + 16 * hb + 4 * q);
      h[4 * q] = v[0];
      h[4 * q + 1] = v[1];
      h[4 * q + 2] = v[2];
      h[4 * q + 3] = v[3];
    }
    float bmax = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) bmax = __builtin_fmaxf(bmax, __builtin_fabsf(h[e]));
    if (to_f32) {
      const int64_t m = row0 + 32 * rb + r;
      if (m < row1) {
        floatx4_t* dst = (floatx4_t*)(p.h_f32 + m * I + hcol);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = floatx4_t{h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]};
        wmax = __builtin_fmaxf(wmax, bmax);
      }
      continue;
    }
    float rcp;
    bool zero;
    const uint32_t sq = block_scale(bmax, gs, rcp, zero);
    const uint32_t lo = e2m1_pack<4>(h, rcp, zero), hi = e2m1_pack<4>(h + 8, rcp, zero);
    const int64_t m = row0 + 32 * rb + r;
    if (m < row1) {
      uint32_t* hc = (uint32_t*)(p.h_codes + m * (I / 2) + hcol / 2);
      hc[0] = lo;
      hc[1] = hi;
      p.h_scales[m * (I / 16) + hcol / 16] = (uint8_t)sq;
      if (p.h_dq) {
        // code times the decoded scale, exact in f16 (the values dq_f16 gives)
        const half2_t sf2 = scale_pair(sq);
        *(half8_t*)(p.h_dq + m * I + hcol) = dequant8(lo, sf2);
        *(half8_t*)(p.h_dq + m * I + hcol + 8) = dequant8(hi, sf2);
      }
    }
  }
  if (to_f32) {
    // the wave's largest |h| (a max: any reduction order gives the same
    // value), at its workgroup's slot (one tile per workgroup)
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) wmax = __builtin_fmaxf(wmax, __shfl_xor(wmax, o, 64));
    const int64_t slot = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (lane == 0 && slot < p.h_amax_n) p.h_amax[slot] = wmax;
  }
}

// gemm_stream32: 32*RB rows x (4 waves x NBW x 32) columns per workgroup; each
// wave streams its NBW 32-column blocks of W over the whole K with two
// half-steps of loads in flight (three register sets; at about 145
// registers three workgroups fit a compute unit, which keeps more bytes in
// flight per compute unit than four workgroups with one half-step each),
// with no shared memory and no barriers.  With skip_bm > 0
// it takes only the rows a skip_bm-row tile launch leaves over at the end of
// each group.
// NT: the tile holds every row of its group, so each weight byte it streams
// is read once in the launch; those loads carry the non-temporal hint, which
// reaches a higher share of the HBM bandwidth than ordinary loads on this chip
// (where several tiles of a group read the same weights, ordinary loads keep
// the repeats in the caches)
// Dependency hooks of the persistent expert kernel (all null elsewhere):
// `signal` is incremented (agent scope, release) once a tile's output is
// stored; before its first A load, a wave waits (agent scope, acquire) until
// `*wait_ctr` reaches `wait_target`, giving up after `spin_limit` polls and
// then recording the failure in `*status`.  The weight loads of the first
// two half-steps are issued before the wait: they do not depend on A.
struct TileSync {
  int32_t* signal = nullptr;
  const int32_t* wait_ctr = nullptr;
  int32_t wait_target = 0;
  int32_t spin_limit = 0;
  int32_t* status = nullptr;
};

// Polls are relaxed; one acquire fence follows the last poll, so the caches
// are invalidated once per wait, not once per poll.
__device__ __forceinline__ void tile_wait(const TileSync& sy) {
  if (!sy.wait_ctr) return;
  int32_t polls = 0;
  while (__hip_atomic_load(sy.wait_ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < sy.wait_target) {
    if (++polls >= sy.spin_limit) {
      // give up: the results are unspecified, the failure is recorded
      if ((threadIdx.x & 63) == 0)
        __hip_atomic_fetch_or(sy.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// One signal per workgroup: every wave's stores are complete before the
// barrier, then one release (cache write-back) and one atomic add.
__device__ __forceinline__ void tile_signal(const TileSync& sy) {
  if (!sy.signal) return;
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(sy.signal, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

template <int NBW, int RB, bool FUSE, bool SPLIT, bool NT>
__device__ __forceinline__ void stream32_tile(const GemmArgs& p, int g, int64_t row0, int64_t row1, int64_t nt,
                                              int wave, int lane, int64_t ks0, int64_t ks1, int split,
                                              const TileSync& sy = TileSync(), float* st = nullptr) {
  static_assert(!FUSE || NBW == 2, "the fused epilogue pairs one gate and one up column block");
  constexpr int BN = 4 * NBW * 32;
  const int c = lane & 31;
  const int kh = lane >> 5;
  const int64_t n0 = nt * BN + wave * NBW * 32;
  // fused: the wave's h column block j, from gate block j and up block I/32 + j
  const int64_t j = nt * 4 + wave;
  if (FUSE ? 64 * j >= p.N : n0 >= p.N) return;
  const int64_t K = p.K;
  const int64_t nks = K / 256;
  const int64_t KB = K / 2, KS = K / 16;

  bool a_valid[RB];
  const uint8_t* a_c[RB];
  const uint8_t* a_s[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t m = row0 + 32 * rb + c;
    a_valid[rb] = m < row1;
    int64_t a_row = a_valid[rb] ? (p.a_row_index ? (int64_t)p.a_row_index[m] : m) : 0;
    a_row = clampv<int64_t>(a_row, 0, p.a_rows > 0 ? p.a_rows - 1 : 0);
    a_c[rb] = p.a_codes + a_row * KB + 32 * kh;
    a_s[rb] = p.a_scales + a_row * KS + 4 * kh;
  }
  // W through one buffer resource per column block: the lane's offset in a
  // VGPR set once, the half-step's offset in an SGPR (no 64-bit address
  // arithmetic per load); the non-temporal bit in the cache-policy field
  const int64_t nb_per_g = (p.N + kTileRows - 1) / kTileRows;
  __amdgpu_buffer_rsrc_t w_rsrc[NBW], w_none[NBW];
#pragma unroll
  for (int cb = 0; cb < NBW; ++cb) {
    int64_t nb = FUSE ? j + cb * (p.N / 64) : n0 / 32 + cb;
    nb = nb < nb_per_g ? nb : nb_per_g - 1;
    w_rsrc[cb] = __builtin_amdgcn_make_buffer_rsrc((void*)(p.w_codes + ((int64_t)g * nb_per_g + nb) * nks * kTileBytes),
                                                   (short)0, (int)(nks * kTileBytes), 0x00020000);
    w_none[cb] = __builtin_amdgcn_make_buffer_rsrc((void*)(p.w_codes + ((int64_t)g * nb_per_g + nb) * nks * kTileBytes),
                                                   (short)0, 0, 0x00020000);
  }
  constexpr int kPol = NT ? 2 : 0;
  const int w_lo = 16 * lane, w_hi = 16 * lane + 1024, w_sc = 4 * lane + 4096;

  floatx16_t acc[RB][NBW];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < NBW; ++cb) acc[rb][cb] = floatx16_t{};

  // operands of one half-step: A codes and scales, W codes and scales
  struct Ops {
    u32x4 a0[RB], a1[RB], w0[NBW], w1[NBW];
    uint32_t as[RB], ws[NBW];
  };
  auto load_a = [&](int64_t hs, Ops& d) {
    const int64_t ks = hs >> 1, h = hs & 1;
    // lanes past the tile's last row load nothing and keep an earlier
    // half-step's values (or the zeros the sets start with): every row of
    // the product depends only on its own A row, and rows >= row1 are never
    // stored.  (Zeroing them made the
    // compiler wait for every load in flight, the next half-steps' weights
    // included, wherever a row block was partial; loading a valid row on
    // every lane instead costs the address unit 64 lanes per load.)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (a_valid[rb]) {
        d.a0[rb] = *(const u32x4*)(a_c[rb] + ks * 128 + 64 * h);
        d.a1[rb] = *(const u32x4*)(a_c[rb] + ks * 128 + 64 * h + 16);
        d.as[rb] = *(const uint32_t*)(a_s[rb] + ks * 16 + 8 * h);
      }
    }
  };
  // dead: the set is never used (the loads of the last two half-steps);
  // its weight loads then go through a resource of no records, where the
  // buffer unit returns zeros without a memory access (on the second GEMM of
  // the decode layer, reloading the last half-step's words instead cost
  // 20 us: a wave cannot end while its loads are in flight).  The choice of
  // resource is a scalar select, no vector work.
  auto load_w = [&](int64_t hs, Ops& d, bool dead) {
    const int ks = (int)(hs >> 1), h = (int)(hs & 1);
    // (uniform by construction; said so, or the compiler keeps them in
    // vector registers and loops over the lanes' distinct values)
    const int so = __builtin_amdgcn_readfirstlane(ks * kTileBytes + 2048 * h);
    const int ss = __builtin_amdgcn_readfirstlane(ks * kTileBytes + 256 * h);
#pragma unroll
    for (int cb = 0; cb < NBW; ++cb) {
      const __amdgpu_buffer_rsrc_t r = dead ? w_none[cb] : w_rsrc[cb];
      d.w0[cb] = __builtin_amdgcn_raw_buffer_load_b128(r, w_lo, so, kPol);
      d.w1[cb] = __builtin_amdgcn_raw_buffer_load_b128(r, w_hi, so, kPol);
      d.ws[cb] = __builtin_amdgcn_raw_buffer_load_b32(r, w_sc, ss, kPol);
    }
  };
  auto load = [&](int64_t hs, Ops& d, bool dead = false) {
    load_a(hs, d);
    load_w(hs, d, dead);
  };
  auto compute = [&](const Ops& o) {
    // the four E4M3 scale bytes of each word, two per conversion (exact:
    // every E4M3 value is an f16 value)
    half2_t wsc[NBW][2], asc[RB][2];
#pragma unroll
    for (int cb = 0; cb < NBW; ++cb) {
      wsc[cb][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(o.ws[cb], 1.0f, false);
      wsc[cb][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(o.ws[cb], 1.0f, true);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      asc[rb][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(o.as[rb], 1.0f, false);
      asc[rb][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(o.as[rb], 1.0f, true);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = j >> 1;    // the block of the substep's 8 codes
      half8_t bf[NBW];
#pragma unroll
      for (int cb = 0; cb < NBW; ++cb) {
        const _Float16 sv = wsc[cb][q >> 1][q & 1];
        bf[cb] = dequant8(j < 4 ? o.w0[cb][j] : o.w1[cb][j - 4], half2_t{sv, sv});
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const _Float16 sv = asc[rb][q >> 1][q & 1];
        const half8_t af = dequant8(j < 4 ? o.a0[rb][j] : o.a1[rb][j - 4], half2_t{sv, sv});
#pragma unroll
        for (int cb = 0; cb < NBW; ++cb) acc[rb][cb] = mfma32(af, bf[cb], acc[rb][cb]);
      }
    }
  };
  // half-steps 2 ks0 .. 2 ks1 - 1 (all of K unless split), two half-steps of
  // loads in flight; the three operand sets rotate (no copy of registers
  // with loads pending)
  const int64_t h0 = 2 * ks0, nhs = 2 * ks1;
  // zeroed once, so that lanes past the last row (which never load A) hold
  // defined values
  Ops s0{}, s1{}, s2{};
  if (sy.wait_ctr) {
    load_w(h0, s0, false);
    load_w(h0 + 1 < nhs ? h0 + 1 : nhs - 1, s1, false);
    tile_wait(sy);
    load_a(h0, s0);
    load_a(h0 + 1 < nhs ? h0 + 1 : nhs - 1, s1);
  } else {
    load(h0, s0);
    load(h0 + 1 < nhs ? h0 + 1 : nhs - 1, s1);
  }
  // (the last two half-steps issue dead loads: no branch around a load)
  auto step = [&](int64_t hs, const Ops& cur, Ops& ld) {
    load(hs + 2 < nhs ? hs + 2 : nhs - 1, ld, hs + 2 >= nhs);
    // the loads go out before the half-step's conversions and MFMAs (the
    // scheduler would otherwise sink them towards their use)
    __builtin_amdgcn_sched_barrier(0);
    compute(cur);
  };
  int64_t hs = h0;
  for (; hs + 3 <= nhs; hs += 3) {
    step(hs, s0, s2);
    step(hs + 1, s1, s0);
    step(hs + 2, s2, s1);
  }
  if (hs < nhs) step(hs, s0, s2);
  if (hs + 1 < nhs) step(hs + 1, s1, s0);

  if constexpr (FUSE) {
    silu_requant_epilogue<RB>(p, acc, g, row0, row1, j, lane, st);
    return;
  }
  if constexpr (SPLIT) {
    // raw partial sums of this split's K range
    float* part = p.ws + (int64_t)split * p.M * p.N;
#pragma unroll
    for (int cb = 0; cb < NBW; ++cb) {
      const int64_t n = n0 + 32 * cb + c;
      if (n >= p.N) continue;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t m = row0 + 32 * rb + acc32_row(i, kh);
          if (m < row1) part[m * p.N + n] = acc[rb][cb][i];
        }
    }
    return;
  }
  const float a_gs = *p.a_gs;
  const int64_t rows = row1 - row0;
#pragma unroll
  for (int cb = 0; cb < NBW; ++cb) {
    const int64_t n = n0 + 32 * cb + c;
    if (n >= p.N) continue;
    const float alpha = alpha_for(p, g, n, a_gs);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // (rows 32 rb + 8 (i / 4) .. + 7: skipped uniformly past the last row)
        if (32 * rb + 8 * (i >> 2) >= rows) continue;
        const int64_t m = row0 + 32 * rb + acc32_row(i, kh);
        if (m < row1) store_out(p, m, n, alpha * acc[rb][cb][i]);
      }
  }
}

// One tile per workgroup, slot-major (the grid is an upper bound; workgroups
// without a tile exit after one pass over the group offsets), or with PERSIST
// a grid of a few workgroups per compute unit, each taking every grid-th
// tile, so that a bound far above the tiles that exist costs no launches.
template <int NBW, int RB, bool FUSE, bool SPLIT = false, bool PERSIST = false>
__global__ __launch_bounds__(256) void gemm_stream32(GemmArgs p, int64_t n_tiles, int skip_bm, int skip_min,
                                                    int64_t total) {
  // the group offsets, staged once per workgroup (all loads in flight
  // together) so that the tile search costs no further global round trips
  __shared__ int32_t s_off[kMaxGroups + 1];
  // the fused epilogue's staging area, 32 rows x kHStride floats per wave
  __shared__ __attribute__((aligned(16))) float s_epi[FUSE ? 4 * 32 * kHStride : 4];
  for (int i = threadIdx.x; i <= p.G; i += blockDim.x) s_off[i] = p.group_offsets[i];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  float* const st = s_epi + (FUSE ? wave * 32 * kHStride : 0);
  // split-K: the grid is splits x (slots x column tiles), split-major
  const int64_t work = SPLIT ? gridDim.x / p.splits : gridDim.x;
  const int split = SPLIT ? (int)(blockIdx.x / work) : 0;
  const int64_t t0 = SPLIT ? (int64_t)blockIdx.x - split * work : (int64_t)blockIdx.x;
  const int64_t nks = p.K / 256;
  const int64_t ks0 = SPLIT ? nks * split / p.splits : 0;
  const int64_t ks1 = SPLIT ? nks * (split + 1) / p.splits : nks;
  if constexpr (!PERSIST) {
    const int64_t slot = t0 / n_tiles;
    const int64_t nt = t0 - slot * n_tiles;
    int g;
    int64_t row0, row1;
    if (!find_tile(s_off, p.G, p.M, slot, 32 * RB, 1, skip_bm, skip_min, g, row0, row1)) return;
    g = __builtin_amdgcn_readfirstlane(g);
    if (row0 == s_off[g] && row1 == s_off[g + 1])
      stream32_tile<NBW, RB, FUSE, SPLIT, true>(p, g, row0, row1, nt, wave, lane, ks0, ks1, split, TileSync(), st);
    else
      stream32_tile<NBW, RB, FUSE, SPLIT, false>(p, g, row0, row1, nt, wave, lane, ks0, ks1, split, TileSync(), st);
  } else {
    // tiles t0, t0 + grid, ... below `total`; slots grow with t, and the
    // tiles that exist come first, so the first missing one ends the loop
    for (int64_t t = t0; t < total; t += work) {
      const int64_t slot = t / n_tiles;
      const int64_t nt = t - slot * n_tiles;
      int g;
      int64_t row0, row1;
      if (!find_tile(s_off, p.G, p.M, slot, 32 * RB, 1, skip_bm, skip_min, g, row0, row1)) return;
      g = __builtin_amdgcn_readfirstlane(g);
      // the lane index made opaque per tile, so that per-lane values are not
      // hoisted out of the loop and kept live across tiles
      int ln = lane;
      asm volatile("" : "+v"(ln));
      if (row0 == s_off[g] && row1 == s_off[g + 1])
        stream32_tile<NBW, RB, FUSE, SPLIT, true>(p, g, row0, row1, nt, wave, ln, ks0, ks1, split, TileSync(), st);
      else
        stream32_tile<NBW, RB, FUSE, SPLIT, false>(p, g, row0, row1, nt, wave, ln, ks0, ks1, split, TileSync(), st);
    }
  }
}

// Number of bm-row tiles over all groups (a last partial tile counts), from
// offsets staged in local memory; every lane gets the result.
__device__ __forceinline__ int64_t count_tiles(const int32_t* __restrict__ offsets, int G, int64_t M, int bm) {
  const int lane = threadIdx.x & 63;
  int64_t total = 0;
  for (int g0 = 0; g0 < G; g0 += 64) {
    const int g = g0 + lane;
    int32_t tiles = 0;
    if (g < G) {
      const int64_t lo = clampv<int64_t>(offsets[g], 0, M);
      int64_t hi = clampv<int64_t>(offsets[g + 1], 0, M);
      if (hi < lo) hi = lo;
      tiles = (int32_t)((hi - lo + bm - 1) / bm);
    }
    total += __builtin_amdgcn_readlane(wave_incl_scan(tiles), 63);
  }
  return total;
}

// ---------------------------------------------------------------------------
// gemm_moe_persistent: the routed experts' MLP in one launch.  A grid of a
// few workgroups per compute unit takes tiles from a device queue (one
// atomic counter) in a fixed order: first every tile of the first GEMM
// (stacked gate_up, SiLU-requant epilogue writing h; slot-major over the
// 32-row slots of every group, then the column tiles), then every tile of
// the second GEMM (down, bf16 y; same slots).  A second-GEMM tile of slot s
// needs the whole h rows of that slot: each first-GEMM workgroup adds 1 to
// done[s] (agent scope, release) once all its waves have stored their h
// blocks, and the second-GEMM waves of slot s issue their first weight
// loads, then wait until done[s] counts all the first GEMM's column tiles
// (relaxed polls, then one agent-scope acquire) before loading h.  So the second GEMM's weight stream starts while the
// first GEMM's last tiles still run, and no launch boundary separates them.
// A tile is taken only by a running workgroup, and every tile of the first
// GEMM is taken before any of the second and never waits, so a waiting tile
// always depends on tiles that running workgroups finish: the launch cannot
// deadlock, whatever the number of resident workgroups.  The waits are
// bounded (spin_limit polls) and a timeout is recorded in ctr[1].
// ctr: [0] queue, [1] status, [2 ..] done per slot; zeroed before the launch.
__global__ __launch_bounds__(256) void gemm_moe_persistent(GemmArgs p1, GemmArgs p2, int32_t* ctr, int64_t n_tiles1,
                                                          int64_t n_tiles2, int64_t max_slots, int32_t spin_limit) {
  __shared__ int32_t s_off[kMaxGroups + 1];
  __shared__ int64_t s_next[2];
  // the fused epilogue's staging area, 32 rows x kHStride floats per wave
  __shared__ __attribute__((aligned(16))) float s_epi[4 * 32 * kHStride];
  for (int i = threadIdx.x; i <= p1.G; i += blockDim.x) s_off[i] = p1.group_offsets[i];
  if (threadIdx.x == 0) s_next[0] = atomicAdd(ctr, 1);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  float* const st = s_epi + wave * 32 * kHStride;
  // (at most the counters there are: offsets that are not a partition of
  // [0, M) cannot index past them)
  const int64_t slots = std::min<int64_t>(count_tiles(s_off, p1.G, p1.M, 32), max_slots);
  const int64_t tiles1 = slots * n_tiles1;
  const int64_t total = tiles1 + slots * n_tiles2;
  const int64_t nks1 = p1.K / 256, nks2 = p2.K / 256;
  const int32_t h_blocks = (int32_t)n_tiles1;          // column tiles of the first GEMM per slot
  int buf = 0;
  int64_t t = s_next[0];
  while (t < total) {
    // the next tile's index is fetched while this one runs
    if (threadIdx.x == 0) s_next[buf ^ 1] = atomicAdd(ctr, 1);
    // the lane index made opaque per tile, so that per-lane values are not
    // hoisted out of the loop and kept live across tiles
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const bool first = t < tiles1;
    const int64_t u = first ? t : t - tiles1;
    const int64_t nt_count = first ? n_tiles1 : n_tiles2;
    const int64_t slot = u / nt_count;
    const int64_t nt = u - slot * nt_count;
    int g;
    int64_t row0, row1;
    if (find_tile(s_off, p1.G, p1.M, slot, 32, 1, 0, 0, g, row0, row1)) {
      g = __builtin_amdgcn_readfirstlane(g);
      const bool whole = row0 == s_off[g] && row1 == s_off[g + 1];
      TileSync sy;
      sy.status = ctr + 1;
      sy.spin_limit = spin_limit;
      if (first) {
        if (whole)
          stream32_tile<2, 1, true, false, true>(p1, g, row0, row1, nt, wave, ln, 0, nks1, 0, sy, st);
        else
          stream32_tile<2, 1, true, false, false>(p1, g, row0, row1, nt, wave, ln, 0, nks1, 0, sy, st);
        // every wave's h stores have reached memory, then one signal for
        // the workgroup's column tile
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        sy.signal = ctr + 2 + slot;
        tile_signal(sy);
      } else {
        sy.wait_ctr = ctr + 2 + slot;
        sy.wait_target = h_blocks;
        if (whole)
          stream32_tile<2, 1, false, false, true>(p2, g, row0, row1, nt, wave, ln, 0, nks2, 0, sy);
        else
          stream32_tile<2, 1, false, false, false>(p2, g, row0, row1, nt, wave, ln, 0, nks2, 0, sy);
      }
    }
    __syncthreads();
    buf ^= 1;
    t = s_next[buf];
  }
}

__global__ void zero_i32(int32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

// Split-K tile for ranges of at most two 256-k steps (32 RB rows, 4 waves x
// NBW column blocks): every load of the range is issued before the first
// MFMA, so a workgroup costs one memory round trip instead of a pipeline
// fill per step.  Loads past the range's end repeat its last half-step and
// are not used; rows past the group's end read its last row (not stored).
// (RB = 4, one workgroup for 128 rows of a group, reads each weight tile
// once instead of four times, but measured slower on the 128-token shared
// expert: every wave then dequantises all 128 rows of A; only RB = 1 is
// launched.)
template <int NBW, int RB>
__device__ __forceinline__ void split_short_tile(const GemmArgs& p, int g, int64_t row0, int64_t row1, int64_t nt,
                                                 int wave, int lane, int64_t ks0, int64_t ks1, int split) {
  constexpr int NH = 4;   // half-steps held at once
  constexpr int BN = 4 * NBW * 32;
  const int c = lane & 31;
  const int kh = lane >> 5;
  const int64_t n0 = nt * BN + wave * NBW * 32;
  if (n0 >= p.N) return;
  const int64_t K = p.K;
  const int64_t nks = K / 256;
  const uint8_t* a_c[RB];
  const uint8_t* a_s[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t m_a = clampv<int64_t>(row0 + 32 * rb + c, row0, row1 - 1);
    int64_t a_row = p.a_row_index ? (int64_t)p.a_row_index[m_a] : m_a;
    a_row = clampv<int64_t>(a_row, 0, p.a_rows > 0 ? p.a_rows - 1 : 0);
    a_c[rb] = p.a_codes + a_row * (K / 2) + 32 * kh;
    a_s[rb] = p.a_scales + a_row * (K / 16) + 4 * kh;
  }
  const int64_t nb_per_g = (p.N + kTileRows - 1) / kTileRows;
  const uint8_t* w_t[NBW];
#pragma unroll
  for (int cb = 0; cb < NBW; ++cb) {
    int64_t nb = n0 / 32 + cb;
    nb = nb < nb_per_g ? nb : nb_per_g - 1;
    w_t[cb] = p.w_codes + ((int64_t)g * nb_per_g + nb) * nks * kTileBytes;
  }
  const int64_t hs0 = 2 * ks0;
  const int nh = (int)(2 * (ks1 - ks0));
  u32x4 a0[NH][RB], a1[NH][RB], w0[NH][NBW], w1[NH][NBW];
  uint32_t as[NH][RB], ws[NH][NBW];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int64_t hs = hs0 + (h < nh ? h : nh - 1);
    const int64_t ks = hs >> 1, hh = hs & 1;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      a0[h][rb] = *(const u32x4*)(a_c[rb] + ks * 128 + 64 * hh);
      a1[h][rb] = *(const u32x4*)(a_c[rb] + ks * 128 + 64 * hh + 16);
      as[h][rb] = *(const uint32_t*)(a_s[rb] + ks * 16 + 8 * hh);
    }
#pragma unroll
    for (int cb = 0; cb < NBW; ++cb) {
      const uint8_t* t = w_t[cb] + ks * kTileBytes;
      w0[h][cb] = *(const u32x4*)(t + 2048 * hh + 16 * lane);
      w1[h][cb] = *(const u32x4*)(t + 2048 * hh + 1024 + 16 * lane);
      ws[h][cb] = *(const uint32_t*)(t + 4096 + 256 * hh + 4 * lane);
    }
  }
  floatx16_t acc[RB][NBW];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < NBW; ++cb) acc[rb][cb] = floatx16_t{};
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    if (h >= nh) break;   // uniform
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      half8_t bf[NBW];
#pragma unroll
      for (int cb = 0; cb < NBW; ++cb)
        bf[cb] = dequant8(j < 4 ? w0[h][cb][j] : w1[h][cb][j - 4], scale_pair(byte_of(ws[h][cb], j >> 1)));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const half8_t af = dequant8(j < 4 ? a0[h][rb][j] : a1[h][rb][j - 4], scale_pair(byte_of(as[h][rb], j >> 1)));
#pragma unroll
        for (int cb = 0; cb < NBW; ++cb) acc[rb][cb] = mfma32(af, bf[cb], acc[rb][cb]);
      }
    }
  }
  float* part = p.ws + (int64_t)split * p.M * p.N;
#pragma unroll
  for (int cb = 0; cb < NBW; ++cb) {
    const int64_t n = n0 + 32 * cb + c;
    if (n >= p.N) continue;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t m = row0 + 32 * rb + acc32_row(i, kh);
        if (m < row1) part[m * p.N + n] = acc[rb][cb][i];
      }
  }
}

template <int NBW, int RB>
__global__ __launch_bounds__(256) void gemm_splitk_short(GemmArgs p, int64_t n_tiles) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t work = gridDim.x / p.splits;
  const int split = (int)(blockIdx.x / work);
  const int64_t t = (int64_t)blockIdx.x - split * work;
  const int64_t slot = t / n_tiles;
  const int64_t nt = t - slot * n_tiles;
  int g;
  int64_t row0, row1;
  if (!find_tile(p.group_offsets, p.G, p.M, slot, 32 * RB, 1, 0, 0, g, row0, row1)) return;
  g = __builtin_amdgcn_readfirstlane(g);
  const int64_t nks = p.K / 256;
  split_short_tile<NBW, RB>(p, g, row0, row1, nt, wave, lane, nks * split / p.splits, nks * (split + 1) / p.splits,
                            split);
}

// Split-K reduction: out[m, n] = alpha(g, n) * (part_0 + part_1 + ...) in
// split order, for the rows m of every group (rows outside all groups are
// left untouched).  Block (x, y): row y, columns 256 x .. 256 x + 255.
// tile_bm > 0: only rows that tiles of tile_bm rows cover (a group's full
// tiles and its last tile when that has at least tile_last_min rows); the
// other rows belong to another kernel's launch.
__global__ __launch_bounds__(256) void splitk_reduce(GemmArgs p) {
  const int64_t m = blockIdx.y;
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= p.N) return;
  // the group holding row m: the last g with offsets[g] <= m (clamped,
  // non-decreasing offsets as find_tile reads them)
  int lo = 0, hi = p.G;                   // answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    const int64_t om = clampv<int64_t>(p.group_offsets[mid], 0, p.M);
    if (om <= m) lo = mid;
    else hi = mid;
  }
  const int64_t g0 = clampv<int64_t>(p.group_offsets[lo], 0, p.M);
  const int64_t g1 = clampv<int64_t>(p.group_offsets[lo + 1], 0, p.M);
  if (m < g0 || m >= g1) return;
  float sum = p.ws[m * p.N + n];
  for (int sp = 1; sp < p.splits; ++sp) sum += p.ws[((int64_t)sp * p.M + m) * p.N + n];
  store_out(p, m, n, alpha_for(p, lo, n, *p.a_gs) * sum);
}

// splitk_reduce for N % 4 == 0, four columns per lane (16-byte loads of the
// partial sums, a wave covering 1 KB of a row per load): the same sums in
// the same order and the same alpha per column.  Block (x, y): row y,
// columns 1024 x .. 1024 x + 1023.  vec: out takes whole 4-column stores
// (16-byte aligned rows for float32, 8-byte for bf16).
__global__ __launch_bounds__(256) void splitk_reduce4(GemmArgs p, bool vec) {
  const int64_t m = blockIdx.y;
  const int64_t n = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (n >= p.N) return;
  int lo = 0, hi = p.G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    const int64_t om = clampv<int64_t>(p.group_offsets[mid], 0, p.M);
    if (om <= m) lo = mid;
    else hi = mid;
  }
  const int64_t g0 = clampv<int64_t>(p.group_offsets[lo], 0, p.M);
  const int64_t g1 = clampv<int64_t>(p.group_offsets[lo + 1], 0, p.M);
  if (m < g0 || m >= g1) return;
  const int64_t plane = p.M * p.N;
  const float* w = p.ws + m * p.N + n;
  floatx4_t sum = *(const floatx4_t*)w;
#pragma unroll 4
  for (int sp = 1; sp < p.splits; ++sp) {
    const floatx4_t t = *(const floatx4_t*)(w + sp * plane);
#pragma unroll
    for (int e = 0; e < 4; ++e) sum[e] += t[e];
  }
  const float a_gs = *p.a_gs;
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = alpha_for(p, lo, n + e, a_gs) * sum[e];
  if (vec) {
    if (p.out_bf16) {
      uint2 o;
      o.x = bf16x2_from_float(v[0], v[1]);
      o.y = bf16x2_from_float(v[2], v[3]);
      *(uint2*)((uint16_t*)p.out + m * p.ld_out + n) = o;
    } else {
      floatx4_t o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = v[e];
      *(floatx4_t*)((float*)p.out + m * p.ld_out + n) = o;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) store_out(p, m, n + e, v[e]);
  }
}

// Split K with SiLU-requant (the first GEMM of the expert MLP): four lanes
// (a DPP quad) per 16-element block of h, each with 4 gate and the matching
// 4 up columns of row m, so that a wave's loads cover 1 KB of contiguous
// partial sums.  Each value is the sum of the raw partial sums in split
// order times alpha, exactly as splitk_reduce stores it; then SiLU(gate) *
// up, the block amax (a max over the quad: order-free), the E4M3 scale and
// the E2M1 codes follow silu_mul_requant's float32 steps, so codes, scales
// and the f16 copy are those of the unfused calls.
__global__ __launch_bounds__(256) void splitk_reduce_silu_requant(GemmArgs p) {
  const int64_t I = p.N / 2, bpr = I / 16;
  const int64_t nq = p.M * bpr * 4;   // a multiple of 4: a quad shares every trip
  const float a_gs = *p.a_gs;
  const float gs = *p.h_gs;
  const int64_t plane = p.M * p.N;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nq; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = t / (bpr * 4);
    const int64_t rem = t - m * bpr * 4;
    const int64_t cb = rem >> 2;
    const int qd = (int)(rem & 3);
    // the group holding row m (as splitk_reduce finds it); the quad agrees
    int lo = 0, hi = p.G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      const int64_t om = clampv<int64_t>(p.group_offsets[mid], 0, p.M);
      if (om <= m) lo = mid;
      else hi = mid;
    }
    const int64_t g0 = clampv<int64_t>(p.group_offsets[lo], 0, p.M);
    const int64_t g1 = clampv<int64_t>(p.group_offsets[lo + 1], 0, p.M);
    if (m < g0 || m >= g1) continue;
    const int64_t n = 16 * cb + 4 * qd;
    const float* wg = p.ws + m * p.N + n;
    floatx4_t sg = *(const floatx4_t*)wg, su = *(const floatx4_t*)(wg + I);
#pragma unroll 4
    for (int sp = 1; sp < p.splits; ++sp) {
      const floatx4_t tg = *(const floatx4_t*)(wg + sp * plane), tu = *(const floatx4_t*)(wg + sp * plane + I);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sg[e] += tg[e];
        su[e] += tu[e];
      }
    }
    const float alpha_g = alpha_for(p, lo, n, a_gs);
    const float alpha_u = alpha_for(p, lo, I + n, a_gs);
    float h[4];
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = silu_mul(alpha_g * sg[e], alpha_u * su[e]);
      amax = __builtin_fmaxf(amax, __builtin_fabsf(h[e]));
    }
    amax = __builtin_fmaxf(amax, dpp_f32<0xB1>(amax));   // quad_perm [1,0,3,2]
    amax = __builtin_fmaxf(amax, dpp_f32<0x4E>(amax));   // quad_perm [2,3,0,1]
    float r;
    bool zero;
    const uint32_t sq = block_scale(amax, gs, r, zero);
    const uint32_t bits = e2m1_pack<2>(h, r, zero);
    *(uint16_t*)(p.h_codes + m * (I / 2) + cb * 8 + 2 * qd) = (uint16_t)bits;
    if (qd == 0) p.h_scales[m * bpr + cb] = (uint8_t)sq;
    if (p.h_dq) {
      const half2_t sf2 = scale_pair(sq);
      uint2 v;
      v.x = __builtin_bit_cast(uint32_t, dequant_pair(bits, 0, sf2));
      v.y = __builtin_bit_cast(uint32_t, dequant_pair(bits, 1, sf2));
      *(uint2*)(p.h_dq + m * I + n) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// gemm_big32: 256 x 256 output tiles for groups with many rows when A comes
// as codes only (with its f16 form the 128-row tiles below run instead), 4
// waves (one per SIMD), each wave all 256 rows x 64 columns = 8 x 2 blocks of 32 x 32
// (256 accumulators, held in the accumulation registers).  A W fragment is
// dequantised once per wave and feeds 8 MFMAs; on gfx950 a 32x32x16 MFMA
// hides only two or three vector instructions, so the dequantisation work
// per MFMA is what the layout minimises.
//  * A (256 rows) is dequantised ONCE per workgroup and half-step into an f16
//    half-tile in LDS: a row is 16 chunks of 16 B, chunk cc holding k
//    [8cc, 8cc + 8) of the half-step, so substep j of k half kh reads chunk
//    8 kh + j.  Chunk cc of row m sits at position cc ^ (m % 16), so the rows
//    a group of lanes reads or writes together fall in distinct banks.  Two
//    buffers, one barrier per half-step.  Wave w converts the 16-byte piece w
//    (chunks 4w..4w+3) of rows lane + 64 pp, pp = 0..3.
//  * A fragments are read from LDS right after their last use in the
//    previous substep, a whole row sweep ahead of their next use.
//  * W goes straight from the tiled layout into registers; the words of the
//    next half-step are loaded into the registers of the current ones as
//    soon as those are dead.
//  * Each of a substep's 16 MFMAs is followed in program order by a slice of
//    vector work: the next substep's W fragments, and in substeps 2..7 the
//    conversion and store of chunks of the next A half-tile.
// Workgroups are mapped to tiles by xcd_tile.
// Workgroup -> (row slot, column tile) for the tile kernels.  The
// hardware sends workgroup b to XCD b % 8; XCD x takes slots x, x + 8, ...,
// each with all its column tiles in turn, so a slot's A rows stay in one
// XCD's L2 while its neighbours' run on the others, and slots without a tile
// (the grid is an upper bound) fall evenly on all XCDs.  The grid holds a
// multiple of 8 slots.
__device__ __forceinline__ void xcd_tile(int64_t bid, int64_t n_tiles, int64_t& slot, int64_t& nt) {
  const int64_t xcd = bid % 8, idx = bid / 8;
  slot = idx / n_tiles * 8 + xcd;
  nt = idx % n_tiles;
}

constexpr int BIG = 256;
constexpr int kAHalfBytes = BIG * 256;           // 64 KiB per f16 half-tile
constexpr int kBigThreads = 256;

__device__ __forceinline__ int swz(int m, int cc) { return m * 256 + ((cc ^ (m & 15)) << 4); }

__global__ __launch_bounds__(kBigThreads, 1) void gemm_big32(GemmArgs p, int64_t n_tiles) {
  constexpr int RB = 8;     // 256 rows per wave
  constexpr int CB = 2;     // 64 columns per wave
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kAHalfBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31;
  const int kh = lane >> 5;

  int64_t slot, nt;
  xcd_tile(blockIdx.x, n_tiles, slot, nt);
  int g;
  int64_t row0, row1;
  if (!find_tile(p.group_offsets, p.G, p.M, slot, BIG, BIG, 0, 0, g, row0, row1)) return;
  g = __builtin_amdgcn_readfirstlane(g);
  const int64_t n0 = nt * BIG;
  const int64_t K = p.K;
  const int64_t nks = K / 256;
  const int64_t KB = K / 2, KS = K / 16;

  // A staging: piece pc = wave of rows lane + 64 pp
  const int pc = wave;
  const uint8_t* a_c[4];
  const uint8_t* a_s[4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    const int64_t m = row0 + lane + 64 * pp;             // always < row1 (full tiles)
    int64_t ar = p.a_row_index ? (int64_t)p.a_row_index[m] : m;
    ar = clampv<int64_t>(ar, 0, p.a_rows - 1);
    a_c[pp] = p.a_codes + ar * KB + 16 * pc;
    a_s[pp] = p.a_scales + ar * KS + 2 * pc;
  }
  const int64_t nb_per_g = (p.N + kTileRows - 1) / kTileRows;
  const uint8_t* w_t[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    int64_t nb = n0 / 32 + wave * CB + cb;
    nb = nb < nb_per_g ? nb : nb_per_g - 1;
    w_t[cb] = p.w_codes + ((int64_t)g * nb_per_g + nb) * nks * kTileBytes;
  }

  floatx16_t acc[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[i][j] = floatx16_t{};

  u32x4 ac[4];
  uint32_t as[4];
  auto a_load = [&](int64_t hs) {
    const int64_t ks = hs >> 1, h = hs & 1;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      ac[pp] = *(const u32x4*)(a_c[pp] + ks * 128 + 64 * h);
      as[pp] = *(const uint16_t*)(a_s[pp] + ks * 16 + 8 * h);
    }
  };
  // W words of the current half-step: w0 (substeps 0-3), w1 (4-7) and the
  // scale word ws; the next half-step's w0 and scale word (wsn) are loaded
  // once substep 3 is done with w0, its w1 during substep 7.
  u32x4 w0[CB], w1[CB];
  uint32_t ws[CB], wsn[CB];
  auto w_load0 = [&](int64_t hs) {
    const int64_t ks = hs >> 1, h = hs & 1;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const uint8_t* t = w_t[cb] + ks * kTileBytes;
      w0[cb] = *(const u32x4*)(t + 2048 * h + 16 * lane);
      wsn[cb] = *(const uint32_t*)(t + 4096 + 256 * h + 4 * lane);
    }
  };
  auto w_load1 = [&](int64_t hs) {
    const int64_t ks = hs >> 1, h = hs & 1;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      w1[cb] = *(const u32x4*)(w_t[cb] + ks * kTileBytes + 2048 * h + 1024 + 16 * lane);
  };

  a_load(0);
  w_load0(0);
  w_load1(0);
#pragma unroll
  for (int pp = 0; pp < 4; ++pp)
#pragma unroll
    for (int d = 0; d < 4; ++d)
      *(half8_t*)(lds + swz(lane + 64 * pp, 4 * pc + d)) =
          dequant8(ac[pp][d], scale_pair((as[pp] >> (8 * (d >> 1))) & 0xFFu));
  half8_t bf[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    ws[cb] = wsn[cb];
    bf[cb] = dequant8(w0[cb][0], scale_pair(byte_of(ws[cb], 0)));
  }
  // LDS byte offsets of this lane's A fragments: row block rb at
  // (32 rb + c) * 256, substep j at chunk_ofs[j]
  const int x = c & 15;
  int chunk_ofs[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) chunk_ofs[j] = ((8 * kh + j) ^ x) << 4;
  __syncthreads();
  const int64_t nhs = 2 * nks;
  for (int64_t hs = 0; hs < nhs; ++hs) {
    const int h = (int)(hs & 1);
    // the last half-step reloads itself instead of reading past K (the
    // words are converted into the unused buffer and never read)
    const int64_t hn = hs + 1 < nhs ? hs + 1 : hs;
    a_load(hn);
    const uint8_t* abuf = lds + h * kAHalfBytes + c * 256;
    uint8_t* anext = lds + (h ^ 1) * kAHalfBytes;
    half8_t af[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) af[rb] = *(const half8_t*)(abuf + rb * 32 * 256 + chunk_ofs[0]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j == 4) w_load0(hn);       // w0's last use was substep 3's dequantisation
      // vector work after the MFMAs, slot s = 2 rb + cb (16 slots):
      //  - W fragments of the next substep: slots 0-9, five parts per column
      //    block (part 0: scale, parts 1-4: one f16 pair each); substep 7
      //    prepares substep 0 of the next half-step;
      //  - in substeps 2..7, chunks of the next A half-tile, three parts per
      //    chunk from slot 6 on (substeps 2-5 three chunks, 6-7 two).
      const int a_first = j < 2 ? 0 : (j < 6 ? 3 * (j - 2) : 12 + 2 * (j - 6));
      const int a_count = j < 2 ? 0 : (j < 6 ? 3 : 2);
      half2_t sfn[CB];
      half8_t bn[CB];
      half2_t asf;
      half8_t aval;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          acc[rb][cb] = mfma32(af[rb], bf[cb], acc[rb][cb]);
          const int s = rb * CB + cb;
          if (s < 10) {  // W fragment of the next substep
            const int wc = s / 5, part = s % 5;
            const uint32_t word = j < 7 ? (j + 1 < 4 ? w0[wc][j + 1] : w1[wc][j + 1 - 4]) : w0[wc][0];
            if (part == 0) {
              sfn[wc] = scale_pair(j < 7 ? byte_of(ws[wc], (j + 1) >> 1) : byte_of(wsn[wc], 0));
            } else {
              const half2_t v = dequant_pair(word, part - 1, sfn[wc]);
              bn[wc][2 * (part - 1)] = v[0];
              bn[wc][2 * (part - 1) + 1] = v[1];
            }
          }
          if (s >= 6 && s - 6 < 3 * a_count) {  // part of a chunk of the next A half-tile
            const int kk = (s - 6) / 3, part = (s - 6) % 3;
            const int chunk = a_first + kk, pp = chunk >> 2, d = chunk & 3;
            if (part == 0) {
              asf = scale_pair((as[pp] >> (8 * (d >> 1))) & 0xFFu);
              const half2_t v0 = dequant_pair(ac[pp][d], 0, asf);
              aval[0] = v0[0];
              aval[1] = v0[1];
            } else if (part == 1) {
              const half2_t v1 = dequant_pair(ac[pp][d], 1, asf);
              const half2_t v2 = dequant_pair(ac[pp][d], 2, asf);
              aval[2] = v1[0];
              aval[3] = v1[1];
              aval[4] = v2[0];
              aval[5] = v2[1];
            } else {
              const half2_t v3 = dequant_pair(ac[pp][d], 3, asf);
              aval[6] = v3[0];
              aval[7] = v3[1];
              *(half8_t*)(anext + swz(lane + 64 * pp, 4 * pc + d)) = aval;
            }
          }
        }
        // af[rb] is dead for this substep: fetch it for the next one
        if (j < 7) af[rb] = *(const half8_t*)(abuf + rb * 32 * 256 + chunk_ofs[j + 1]);
      }
      if (j == 7) w_load1(hn);       // w1's last use was substep 6's dequantisation
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) bf[cb] = bn[cb];
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) ws[cb] = wsn[cb];
    __syncthreads();
  }

  const float a_gs = *p.a_gs;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int64_t n = n0 + (wave * CB + cb) * 32 + c;
    if (n >= p.N) continue;
    const float alpha = alpha_for(p, g, n, a_gs);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        store_out(p, row0 + rb * 32 + acc32_row(i, kh), n, alpha * acc[rb][cb][i]);
  }
}

// ---------------------------------------------------------------------------
// big_dq_tile: one tile of up to 128 rows x 256 columns when A also comes in
// its exactly dequantised f16 form (a_dq).  A half-tiles go from global
// memory straight into local memory (buffer loads into LDS, 1 KiB = four
// 256-byte rows per wave instruction), so A costs the waves neither vector
// registers nor conversion work, and the vector unit only dequantises W.
//  * The tile has R = 32 RB rows (RB = 4, or 2 or 1 for a group's last tile
//    of at most 64 or 32 rows); each wave computes all R rows x 64 columns
//    (RB x 2 blocks of 32 x 32).  The four waves copy the rows, wave w
//    taking rows 8 RB w .. 8 RB w + 8 RB - 1 in 2 RB copies: copy i fills
//    rows 8 RB w + 4 i .. +3, lane l writing physical chunk l % 16 of row
//    8 RB w + 4 i + l / 16.  That chunk holds logical chunk (l % 16) ^ (row %
//    16) (the swizzle of gemm_big32), so the lane reads those 16 bytes of
//    the row.  Rows past the group's end copy its last row; their results
//    are not stored.
//  * The next half-tile's copies are spread over substeps 0-3.  W words are
//    loaded two half-steps ahead (PF = 2: after the half-step's copies, at
//    substep 4, into three register sets that rotate) or one (PF = 1: at
//    substep 0, into a second set); the barrier at the end of a half-step
//    waits for the copies only.
// Output of one wave's block of a tile (RB row blocks of 32, two
// column blocks of 32) staged through LDS, 32 rows at a time, so that every
// lane stores 16 contiguous bytes of one row: a quarter (f32) or an eighth
// (bf16) of the store instructions of one element per lane, and no address
// arithmetic per element.  Values and rounding are those of store_out.  The
// caller guarantees that the tile's LDS is free (every wave is past the main
// loop's last barrier), that out is 16-byte aligned and that ld_out and N are
// multiples of 8.
constexpr int kEpiStride = 68;   // floats per staged row: 64, plus 4 to shift the next row's banks
template <int RB>
__device__ __forceinline__ void store_block_vec(const GemmArgs& p, uint8_t* lds, const floatx16_t (&acc)[RB][2],
                                                const float (&alpha)[2], int64_t row0, int64_t row1, int64_t nw,
                                                int wave, int lane) {
  const int c = lane & 31, kh = lane >> 5;
  float* st = (float*)lds + wave * 32 * kEpiStride;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) st[acc32_row(i, kh) * kEpiStride + 32 * cb + c] = alpha[cb] * acc[rb][cb][i];
    // one wave's LDS operations complete in issue order: the reads below see
    // the writes above, and the next row block's writes follow these reads
    const int64_t mb = row0 + 32 * rb;
    if (p.out_bf16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;     // 32 rows x 8 chunks of 8 columns
        const int r = e >> 3, ch = e & 7;
        const floatx4_t lo = *(const floatx4_t*)(st + r * kEpiStride + 8 * ch);
        const floatx4_t hi = *(const floatx4_t*)(st + r * kEpiStride + 8 * ch + 4);
        const int64_t m = mb + r, n = nw + 8 * ch;
        if (m < row1 && n < p.N) {
          u32x4 w;
          w[0] = bf16x2_from_float(lo[0], lo[1]);
          w[1] = bf16x2_from_float(lo[2], lo[3]);
          w[2] = bf16x2_from_float(hi[0], hi[1]);
          w[3] = bf16x2_from_float(hi[2], hi[3]);
          *(u32x4*)((uint16_t*)p.out + m * p.ld_out + n) = w;
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int e = lane + 64 * q;     // 32 rows x 16 chunks of 4 columns
        const int r = e >> 4, ch = e & 15;
        const floatx4_t v = *(const floatx4_t*)(st + r * kEpiStride + 4 * ch);
        const int64_t m = mb + r, n = nw + 4 * ch;
        if (m < row1 && n < p.N) *(floatx4_t*)((float*)p.out + m * p.ld_out + n) = v;
      }
    }
  }
}

// s_waitcnt immediate: vmcnt 6, expcnt 0, lgkmcnt 0
constexpr int kVmcnt6 = 6;
constexpr int BIG4 = 128;
constexpr int kA4HalfBytes = BIG4 * 256;   // 32 KiB per f16 half-tile
template <int RB, bool FUSE, bool SPLIT = false, int PF = 2>
__device__ __forceinline__ void big_dq_tile(const GemmArgs& p, uint8_t* lds, int g, int64_t row0, int64_t row1,
                                            int64_t n0, int wave, int lane, int64_t hs0 = 0, int64_t hs1 = -1,
                                            int split = 0) {
  constexpr int CB = 2;            // 64 columns per wave
  constexpr int NC = 2 * RB;       // copies per wave and half-step
  const int c = lane & 31;
  const int kh = lane >> 5;
  const int64_t K = p.K;
  const int64_t nks = K / 256;

  // byte offsets in a_dq of this lane's 16 bytes of each copy, less the
  // half-step's k offset (the host guarantees a_rows * K * 2 < 2^32)
  // (lane l < 8 RB looks up the stored row of the wave's row l once; the
  // copies take it from that lane)
  int32_t ar_l;
  {
    const int64_t m = clampv<int64_t>(row0 + 8 * RB * wave + (lane < 8 * RB ? lane : 0), row0, row1 - 1);
    const int64_t ar = p.a_row_index ? (int64_t)p.a_row_index[m] : m;
    ar_l = (int32_t)clampv<int64_t>(ar, 0, p.a_rows - 1);
  }
  uint32_t a_off[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int r = 4 * i + (lane >> 4);             // row within the wave's rows
    const int tr = 8 * RB * wave + r;               // row within the tile (sets the swizzle)
    const uint32_t ar = (uint32_t)__shfl(ar_l, r, 64);
    a_off[i] = ar * (uint32_t)K * 2u + 16u * (uint32_t)((lane & 15) ^ (tr & 15));
  }
  // A through a buffer resource: the lane's 32-bit offset in a VGPR, the
  // half-step's k offset in an SGPR
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.a_dq, (short)0, (int)(uint32_t)(p.a_rows * K * 2), 0x00020000);
  auto a_copy = [&](int64_t hs, int buf, int i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        a_rsrc, (__attribute__((address_space(3))) void*)(lds + buf * kA4HalfBytes + (8 * RB * wave + 4 * i) * 256),
        16, (int)a_off[i], (int)(hs * 256), 0, 0);
  };

  const int64_t nb_per_g = (p.N + kTileRows - 1) / kTileRows;
  // fused: the wave's h column block j, from gate block j and up block I/32 + j
  const int64_t j = n0 / 64 + wave;
  __amdgpu_buffer_rsrc_t w_rsrc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    int64_t nb = FUSE ? j + cb * (p.N / 64) : n0 / 32 + wave * CB + cb;
    nb = nb < nb_per_g ? nb : nb_per_g - 1;
    w_rsrc[cb] = __builtin_amdgcn_make_buffer_rsrc((void*)(p.w_codes + ((int64_t)g * nb_per_g + nb) * nks * kTileBytes),
                                                   (short)0, (int)(nks * kTileBytes), 0x00020000);
  }
  const int w_lo = 16 * lane, w_hi = 16 * lane + 1024, w_sc = 4 * lane + 4096;
  // W words of a half-step: w0 (substeps 0-3), w1 (4-7), scale word ws
  struct WWords {
    u32x4 w0[CB], w1[CB];
    uint32_t ws[CB];
  };
  auto w_load = [&](int64_t hs, WWords& d) {
    const int ks = (int)(hs >> 1), h = (int)(hs & 1);
    const int so = ks * kTileBytes + 2048 * h, ss = ks * kTileBytes + 256 * h;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      d.w0[cb] = __builtin_amdgcn_raw_buffer_load_b128(w_rsrc[cb], w_lo, so, 0);
      d.w1[cb] = __builtin_amdgcn_raw_buffer_load_b128(w_rsrc[cb], w_hi, so, 0);
      d.ws[cb] = __builtin_amdgcn_raw_buffer_load_b32(w_rsrc[cb], w_sc, ss, 0);
    }
  };

  floatx16_t acc[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[i][j] = floatx16_t{};

  // half-steps hs0 .. hs1 - 1 (all of K unless split); hs0 is in buffer 0.
  // PF = 1: a half-step's W words are loaded at the start of the one before
  // (into nxt).  PF = 2: two half-steps ahead, after that half-step's A
  // copies (at its substep 4), into nxt and far alternately; the wait at the
  // end of a half-step then leaves those six loads in flight.
  if (hs1 < 0) hs1 = 2 * nks;
  WWords cur, nxt, far;
#pragma unroll
  for (int i = 0; i < NC; ++i) a_copy(hs0, 0, i);
  w_load(hs0, cur);
  if constexpr (PF == 2) w_load(hs0 + 1 < hs1 ? hs0 + 1 : hs0, nxt);
  half8_t bf[CB];
  // the half-step's four scale bytes per column block as two f16 pairs
  half2_t sc_lo[CB], sc_hi[CB], sc_n[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    sc_lo[cb] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cur.ws[cb], 1.0f, false);
    sc_hi[cb] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cur.ws[cb], 1.0f, true);
    sc_n[cb] = sc_lo[cb];
    bf[cb] = dequant8(cur.w0[cb][0], half2_t{sc_lo[cb][0], sc_lo[cb][0]});
  }
  const int x = c & 15;
  int chunk_ofs[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) chunk_ofs[j] = ((8 * kh + j) ^ x) << 4;
  // this wave's copies of the first half-tile have landed (PF = 2: the six
  // loads of the second half-step's W words may still be in flight)
  if constexpr (PF == 2)
    __builtin_amdgcn_s_waitcnt(kVmcnt6);
  else
    __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // one half-step: cu holds its W words, nx the next half-step's (PF = 1:
  // loaded here), fa receives the words two half-steps ahead (PF = 2)
  auto half_step = [&](int64_t hs, const WWords& cu, WWords& nx, WWords& fa) __attribute__((always_inline)) {
    const int h = (int)((hs - hs0) & 1);
    // the last half-step reloads itself (into the unused buffer and registers)
    const int64_t hn = hs + 1 < hs1 ? hs + 1 : hs;
    if constexpr (PF == 1) w_load(hn, nx);
    const uint8_t* abuf = lds + h * kA4HalfBytes + c * 256;
    half8_t af[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) af[rb] = *(const half8_t*)(abuf + rb * 32 * 256 + chunk_ofs[0]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (PF == 2) {
        // after the A copies of substeps 0-3 (sched_barrier keeps the order)
        if (j == 4) w_load(hs + 2 < hs1 ? hs + 2 : hs1 - 1, fa);
      }
      half2_t sfn[CB];
      half8_t bn[CB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          acc[rb][cb] = mfma32(af[rb], bf[cb], acc[rb][cb]);
          const int s = rb * CB + cb;
          // the next half-tile's copies: NC / 4 per substep in substeps 0-3
          // after slots 3, 7, ... (RB = 1: one in substeps 0 and 1)
          if constexpr (RB >= 2) {
            if (j < 4 && (s & 3) == 3) a_copy(hn, h ^ 1, j * (RB / 2) + (s >> 2));
          } else {
            if (j < 2 && s == 1) a_copy(hn, h ^ 1, j);
          }
        }
        // af[rb] is dead for this substep: fetch it for the next one
        if (j < 7) af[rb] = *(const half8_t*)(abuf + rb * 32 * 256 + chunk_ofs[j + 1]);
      }
      // W fragments of the next substep (substep 7 prepares substep 0 of the
      // next half-step), interleaved by the scheduler with the MFMAs above
#pragma unroll
      for (int wc = 0; wc < CB; ++wc) {
        const uint32_t word = j < 7 ? (j + 1 < 4 ? cu.w0[wc][j + 1] : cu.w1[wc][j + 1 - 4]) : nx.w0[wc][0];
        if (j == 6) sc_n[wc] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(nx.ws[wc], 1.0f, false);
        const half2_t sp = j < 7 ? (((j + 1) >> 1) < 2 ? sc_lo[wc] : sc_hi[wc]) : sc_n[wc];
        const _Float16 sv = j < 7 ? sp[((j + 1) >> 1) & 1] : sp[0];
        sfn[wc] = half2_t{sv, sv};
#pragma unroll
        for (int part = 0; part < 4; ++part) {
          const half2_t v = dequant_pair(word, part, sfn[wc]);
          bn[wc][2 * part] = v[0];
          bn[wc][2 * part + 1] = v[1];
        }
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) bf[cb] = bn[cb];
      // keep each substep's loads and conversions among its own MFMAs (the
      // scheduler would otherwise move the loads towards their first use)
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      sc_lo[cb] = sc_n[cb];
      sc_hi[cb] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(nx.ws[cb], 1.0f, true);
    }
    // this wave's copies of the next half-tile have landed
    if constexpr (PF == 2)
      __builtin_amdgcn_s_waitcnt(kVmcnt6);
    else
      __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  if constexpr (PF == 2) {
    // the three register sets rotate: unrolled by three, so that no set is
    // ever copied (a copy of a set with loads in flight would wait for them)
    int64_t hs = hs0;
    for (; hs + 3 <= hs1; hs += 3) {
      half_step(hs, cur, nxt, far);
      half_step(hs + 1, nxt, far, cur);
      half_step(hs + 2, far, cur, nxt);
    }
    if (hs < hs1) half_step(hs, cur, nxt, far);
    if (hs + 1 < hs1) half_step(hs + 1, nxt, far, cur);
  } else {
    for (int64_t hs = hs0; hs < hs1; ++hs) {
      half_step(hs, cur, nxt, far);
      cur = nxt;
    }
  }

  if constexpr (FUSE) {
    silu_requant_epilogue<RB>(p, acc, g, row0, row1, j, lane, (float*)lds + wave * 32 * kHStride);
    return;
  }
  if constexpr (SPLIT) {
    // raw partial sums of this split's k range, float32 [M, N] per split
    GemmArgs q = p;
    q.out = p.ws + (int64_t)split * p.M * p.N;
    q.out_bf16 = false;
    q.ld_out = p.N;
    const float one[CB] = {1.0f, 1.0f};
    if ((p.N & 7) == 0) {
      store_block_vec<RB>(q, lds, acc, one, row0, row1, n0 + wave * CB * 32, wave, lane);
    } else {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int64_t n = n0 + (wave * CB + cb) * 32 + c;
        if (n >= p.N) continue;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int64_t m = row0 + rb * 32 + acc32_row(i, kh);
            if (m < row1) store_out(q, m, n, acc[rb][cb][i]);
          }
      }
    }
    return;
  }
  const float a_gs = *p.a_gs;
  if (((uintptr_t)p.out & 15) == 0 && (p.ld_out & 7) == 0 && (p.N & 7) == 0) {
    float alpha[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int64_t n = n0 + (wave * CB + cb) * 32 + c;
      alpha[cb] = n < p.N ? alpha_for(p, g, n, a_gs) : 0.0f;
    }
    store_block_vec<RB>(p, lds, acc, alpha, row0, row1, n0 + wave * CB * 32, wave, lane);
    return;
  }
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int64_t n = n0 + (wave * CB + cb) * 32 + c;
    if (n >= p.N) continue;
    const float alpha = alpha_for(p, g, n, a_gs);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t m = row0 + rb * 32 + acc32_row(i, kh);
        if (m < row1) store_out(p, m, n, alpha * acc[rb][cb][i]);
      }
  }
}

// gemm_big32_dq4: the 128 x 256 tiles (RB = 4: each wave 128 rows x 64
// columns, 128 accumulators), at most 256 registers per lane and 64 KiB of
// local memory, so two workgroups share a compute unit: each SIMD runs one
// wave of each, and while one workgroup waits at its per-half-step barrier,
// or runs a tile's prologue or epilogue, the other's waves keep the matrix
// core busy.  Every group's rows are cut into 128-row tiles, the last one 32,
// 64 or 128 rows high (the smallest that holds it).
template <bool FUSE>
__global__ __launch_bounds__(kBigThreads, 2) void gemm_big32_dq4(GemmArgs p, int64_t n_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kA4HalfBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t slot, nt;
  xcd_tile((int64_t)blockIdx.x, n_tiles, slot, nt);
  int g;
  int64_t row0, row1;
  if (!find_tile_batched(p.group_offsets, p.G, p.M, slot, BIG4, 1, 0, 0, g, row0, row1)) return;
  g = __builtin_amdgcn_readfirstlane(g);
  row0 = __builtin_amdgcn_readfirstlane((int)row0);
  row1 = __builtin_amdgcn_readfirstlane((int)row1);
  const int64_t rows = row1 - row0;
  if (rows > 64)
    big_dq_tile<4, FUSE>(p, lds, g, row0, row1, nt * BIG, wave, lane);
  else if (rows > 32)
    big_dq_tile<2, FUSE>(p, lds, g, row0, row1, nt * BIG, wave, lane);
  else
    big_dq_tile<1, FUSE>(p, lds, g, row0, row1, nt * BIG, wave, lane);
}

// One group (G = 1) with few tiles for the chip, A in f16 form, K split:
// block b takes k range b / (n_slots n_tiles), then row slot and column tile
// of the 128 x 256 tile loop above (A through local memory, each weight tile
// read once per 128 rows), writing raw partial sums that splitk_reduce adds
// in range order.  No tile search: the group is rows [offsets[0],
// offsets[1]), cut into 128-row slots (the last one partial).
__global__ __launch_bounds__(kBigThreads, 2) void gemm_dq4_split(GemmArgs p, int64_t n_slots, int64_t n_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kA4HalfBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t per_split = n_slots * n_tiles;
  const int split = (int)(blockIdx.x / per_split);
  const int64_t rem = (int64_t)blockIdx.x - split * per_split;
  const int64_t slot = rem / n_tiles, nt = rem - slot * n_tiles;
  const int64_t g0 = clampv<int64_t>(p.group_offsets[0], 0, p.M);
  const int64_t g1 = clampv<int64_t>(p.group_offsets[1], g0, p.M);
  const int64_t row0 = g0 + slot * BIG4;
  const int64_t row1 = row0 + BIG4 < g1 ? row0 + BIG4 : g1;
  if (row1 <= row0) return;
  const int64_t nks = p.K / 256;
  const int64_t hs0 = 2 * (nks * split / p.splits), hs1 = 2 * (nks * (split + 1) / p.splits);
  if (row1 - row0 > 64)
    big_dq_tile<4, false, true>(p, lds, 0, row0, row1, nt * BIG, wave, lane, hs0, hs1, split);
  else if (row1 - row0 > 32)
    big_dq_tile<2, false, true>(p, lds, 0, row0, row1, nt * BIG, wave, lane, hs0, hs1, split);
  else
    big_dq_tile<1, false, true>(p, lds, 0, row0, row1, nt * BIG, wave, lane, hs0, hs1, split);
}

// whether launch_tiled, given A in f16 form and a split-K workspace, runs
// one group of at most 128 rows on gemm_dq4_split
bool gemm_small_split(int64_t G, int64_t M, bool tiled) { return tiled && G == 1 && M >= 1 && M <= BIG4; }

// ---------------------------------------------------------------------------
// The matrix-core tiles from 32 rows per group on average (16 where K <=
// 4096, the second GEMM of the layer); below that the streaming kernel,
// which reads each group's weights once per 32-row slot from HBM, is faster.
// Measured on the routed layer (384 experts, top-6): T = 2048 3.98 -> 3.16
// ms and T = 3072 4.41 -> 3.48 ms against the 64-row rule of the 256-row
// tiles; at T = 1024 (16 rows) the tiles gain on the second GEMM (1.01 ->
// 0.90 ms) and lose on the first (1.72 -> 1.75 ms)
bool gemm_uses_big_tiles(int64_t G, int64_t M, int64_t K, bool tiled) {
  return tiled && M >= BIG && M >= (K > 4096 ? 32 : 16) * G;
}

// The raw partial sums of a split-K GEMM into a.ws (splits x [M, N] float32,
// split-major): one group with A in f16 form on the 128-row tiles, else the
// weight-streaming kernels (short ranges where 16 of them cover K).
hipError_t launch_split_partials(const GemmArgs& a, hipStream_t s) {
  if (a.a_dq && a.G == 1) {
    const int64_t n_tiles = (a.N + BIG - 1) / BIG;
    const int64_t n_slots = (a.M + BIG4 - 1) / BIG4;
    hipLaunchKernelGGL(gemm_dq4_split, dim3((unsigned)(n_slots * n_tiles * a.splits)), dim3(kBigThreads), 0, s, a,
                       n_slots, n_tiles);
    return hipGetLastError();
  }
  constexpr int NBW = 2;
  const int64_t n_tiles = (a.N + 4 * NBW * 32 - 1) / (4 * NBW * 32);
  const int64_t work = ((a.M + 31) / 32 + a.G) * n_tiles;
  const int64_t nks = a.K / 256;
  if ((nks + a.splits - 1) / a.splits <= 2)
    hipLaunchKernelGGL((gemm_splitk_short<NBW, 1>), dim3((unsigned)(work * a.splits)), dim3(256), 0, s, a, n_tiles);
  else
    hipLaunchKernelGGL((gemm_stream32<NBW, 1, false, true>), dim3((unsigned)(work * a.splits)), dim3(256), 0, s, a,
                       n_tiles, 0, 0, work);
  return hipGetLastError();
}

template <bool FUSE>
hipError_t launch_tiled(const GemmArgs& a, hipStream_t s) {
  if (FUSE && a.h_f32) {
    // float32 h: the per-wave maxima start at zero (waves without rows leave
    // their entries so); no split-K in this mode
    if (a.splits > 1 || !a.h_amax) return hipErrorInvalidValue;
    hipLaunchKernelGGL(zero_i32, dim3((unsigned)std::min<int64_t>((a.h_amax_n + 255) / 256, 1024)), dim3(256), 0, s,
                       (int32_t*)a.h_amax, a.h_amax_n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.splits > 1 && a.ws && (a.G == 1 && a.a_dq || !gemm_uses_big_tiles(a.G, a.M, a.K, true))) {
    // few workgroups for the chip (gemm_splitk_splits): K split, then the
    // partial sums reduced in split order, to the output or (fused) through
    // SiLU-requant
    hipError_t e = launch_split_partials(a, s);
    if (e != hipSuccess) return e;
    if constexpr (FUSE) {
      // 64-lane workgroups: a few per compute unit even for a 128-row call
      const int64_t nq = a.M * (a.N / 2 / 16) * 4;
      const int64_t grid = std::min<int64_t>((nq + 63) / 64, 1 << 20);
      hipLaunchKernelGGL(splitk_reduce_silu_requant, dim3((unsigned)grid), dim3(64), 0, s, a);
    } else if (a.N % 4 == 0) {
      const bool vec = a.ld_out % 4 == 0 && ((uintptr_t)a.out & (a.out_bf16 ? 7 : 15)) == 0;
      hipLaunchKernelGGL(splitk_reduce4, dim3((unsigned)((a.N + 1023) / 1024), (unsigned)a.M), dim3(256), 0, s, a,
                         vec);
    } else {
      hipLaunchKernelGGL(splitk_reduce, dim3((unsigned)((a.N + 255) / 256), (unsigned)a.M), dim3(256), 0, s, a);
    }
    return hipGetLastError();
  }
  // a workgroup covers 256 weight rows: 256 output columns, or (fused) 128
  // columns of h from 128 gate and 128 up rows
  if (gemm_uses_big_tiles(a.G, a.M, a.K, true) && (a.a_dq || !FUSE)) {
    // many rows per group.  Tile counts are upper bounds (the group sizes are
    // on the device); workgroups without a tile exit.
    const int64_t n_tiles = (a.N + BIG - 1) / BIG;
    if (a.a_dq) {
      // A in f16 form: 128-row tiles, two workgroups per compute unit, each
      // group's last tile 32, 64 or 128 rows high
      const int64_t slots4 = (a.M / BIG4 + a.G + 7) / 8 * 8;
      hipLaunchKernelGGL(gemm_big32_dq4<FUSE>, dim3((unsigned)(slots4 * n_tiles)), dim3(kBigThreads), 0, s, a,
                         n_tiles);
      return hipGetLastError();
    }
    if constexpr (!FUSE) {
      // A as codes only: full 256-row tiles (gemm_big32), the rows each
      // group leaves over on the streaming kernel, persistent: three
      // workgroups per compute unit (about 150 registers with two half-steps
      // of loads in flight)
      constexpr int NBW = 2, RB = 1;
      const int64_t n_tiles_s = (a.N + 4 * NBW * 32 - 1) / (4 * NBW * 32);
      // a group leaves fewer than 256 rows over: at most 8 32-row tiles per
      // group, and at most M / 32 + G in all
      const int64_t work_s = std::min<int64_t>((a.M + 32 * RB - 1) / (32 * RB) + a.G, 8 * a.G) * n_tiles_s;
      const int64_t grid_s = std::min<int64_t>(work_s, 768);
      hipLaunchKernelGGL((gemm_stream32<NBW, RB, false, false, true>), dim3((unsigned)grid_s), dim3(256), 0, s, a,
                         n_tiles_s, BIG, BIG, work_s);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int64_t slots = (a.M / BIG + 7) / 8 * 8;
      hipLaunchKernelGGL(gemm_big32, dim3((unsigned)(slots * n_tiles)), dim3(kBigThreads), 0, s, a, n_tiles);
    }
    return hipGetLastError();
  }
  constexpr int NBW = 2;
  const int64_t n_tiles = (a.N + 4 * NBW * 32 - 1) / (4 * NBW * 32);
  const int64_t work = ((a.M + 31) / 32 + a.G) * n_tiles;
  hipLaunchKernelGGL((gemm_stream32<NBW, 1, FUSE>), dim3((unsigned)work), dim3(256), 0, s, a, n_tiles, 0, 0, work);
  return hipGetLastError();
}

int64_t moe_persistent_counters(int64_t G, int64_t M) { return 2 + (M + 31) / 32 + G; }

int64_t gemm_silu_f32_amax_slots(int64_t G, int64_t M, int64_t I) {
  // the fused launches of launch_tiled: 128-row tiles (slots4 x n_tiles
  // workgroups) or the streaming kernel (one per 32-row slot and column tile)
  const int64_t n_tiles = (2 * I + 255) / 256;
  const int64_t slots4 = (M / BIG4 + G + 7) / 8 * 8;
  const int64_t slots32 = (M + 31) / 32 + G;
  // (a multiple of 8, so that nvfp4_global_scale can reduce the array)
  return (4 * n_tiles * std::max(slots4, slots32) + 7) / 8 * 8;
}

hipError_t launch_moe_persistent(const GemmArgs& l1, const GemmArgs& l2, int32_t* ctr, int32_t spin_limit,
                                 hipStream_t s) {
  if (l1.M == 0) return hipSuccess;
  if (l1.G < 1 || l1.G > kMaxGroups) return hipErrorInvalidValue;
  const int64_t n_ctr = moe_persistent_counters(l1.G, l1.M);
  hipLaunchKernelGGL(zero_i32, dim3((unsigned)std::min<int64_t>((n_ctr + 255) / 256, 1024)), dim3(256), 0, s, ctr,
                     n_ctr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // three workgroups per compute unit (the streaming tiles' register use)
  static int cus = 0;
  if (!cus) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
        hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  constexpr int NBW = 2;
  const int64_t n_tiles1 = (l1.N + 4 * NBW * 32 - 1) / (4 * NBW * 32);
  const int64_t n_tiles2 = (l2.N + 4 * NBW * 32 - 1) / (4 * NBW * 32);
  hipLaunchKernelGGL(gemm_moe_persistent, dim3((unsigned)(3 * cus)), dim3(256), 0, s, l1, l2, ctr, n_tiles1,
                     n_tiles2, n_ctr - 2, spin_limit);
  return hipGetLastError();
}

int32_t gemm_splitk_splits(int64_t G, int64_t M, int64_t N, int64_t K, bool tiled) {
  // the streaming path with fewer than 512 workgroups (two per compute unit)
  // splits K; the reduction's grid has one row per block
  if (!tiled || M < 1 || M > 65535 || K % 256) return 1;
  if (gemm_uses_big_tiles(G, M, K, tiled)) {
    // one group whose 128-row tiles would leave a compute unit without its
    // second workgroup: about 512 workgroups over k ranges of at least one
    // 256-k step (used with the f16 form of A only)
    if (G != 1) return 1;
    const int64_t tiles = ((M + BIG4 - 1) / BIG4) * ((N + BIG - 1) / BIG);
    if (tiles > 256) return 1;
    const int64_t sp = std::min<int64_t>(std::min<int64_t>(512 / tiles, K / 256), 8);
    return sp > 1 ? (int32_t)sp : 1;
  }
  if (gemm_small_split(G, M, tiled)) {
    // one group of at most 128 rows (with A in f16 form on the 128-row
    // tiles): ranges for about 176 tiles, one per compute unit.  Measured on
    // the shared expert (128 rows): 7 ranges of the first GEMM take 25.0 us
    // against 29.8 us at 14 (more partial sums to write and add) and 28.0 at
    // 5; the second GEMM is flat from 2 to 8 ranges
    const int64_t sp = std::min<int64_t>(std::min<int64_t>(176 / ((N + BIG - 1) / BIG), K / 256), 16);
    return sp > 1 ? (int32_t)sp : 1;
  }
  const int64_t base = ((M + 31) / 32 + G) * ((N + 255) / 256);
  if (base >= 512) return 1;
  // ranges of at most two 256-k steps where 16 of them cover K (the
  // short-range kernel), else 16 ranges
  const int64_t nks = K / 256;
  const int64_t sp = std::min<int64_t>(16, (nks + 1) / 2);
  return sp > 1 ? (int32_t)sp : 1;
}

size_t gemm_splitk_bytes(int64_t G, int64_t M, int64_t N, int64_t K, bool tiled) {
  const int32_t sp = gemm_splitk_splits(G, M, N, K, tiled);
  return sp > 1 ? (size_t)sp * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  if (a.G < 1 || a.G > kMaxGroups) return hipErrorInvalidValue;  // the kernels stage at most kMaxGroups offsets
  if (a.w_tiled) return a.fuse ? launch_tiled<true>(a, s) : launch_tiled<false>(a, s);
  if (a.fuse) return hipErrorInvalidValue;  // the fused epilogue runs on the tiled kernels only
  if (a.M >= (int64_t)64 * a.G && a.K % TBK == 0) {
    const int64_t n_tiles = (a.N + TBN - 1) / TBN;
    const int64_t slots = (a.M + TBM - 1) / TBM + a.G;
    hipLaunchKernelGGL(gemm_tile16, dim3((unsigned)(slots * n_tiles)), dim3(256), 0, s, a, n_tiles);
  } else {
    constexpr int NBW = 4;
    const int64_t n_tiles = (a.N + 4 * NBW * 16 - 1) / (4 * NBW * 16);
    const int64_t slots = (a.M + 15) / 16 + a.G;
    hipLaunchKernelGGL((gemm_stream16<NBW, 1>), dim3((unsigned)(slots * n_tiles)), dim3(256), 0, s, a, n_tiles, 0);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
