// Top-k routing and the stable group-by-expert permutation.
#include "nvfp4_device.hpp"
#include "launch.hpp"

namespace nvfp4 {

constexpr int kMaxPerLane = 16;   // 64 lanes x 16 = NVFP4_MAX_EXPERTS logits per wave

// One wave per token.  Lane l holds logits l, l+64, l+128, ...; k rounds of a
// wave-wide arg-max pick the experts in slot order.  "Better" means a larger
// logit, or an equal logit with a lower expert id, so the selection does not
// depend on evaluation order.  Lane 0 then forms the softmax over the k
// selected logits in slot order.
// ns > 0: each token's row of ids/w has k + ns slots; slots k .. k+ns-1 are
// the always-on shared experts E .. E+ns-1 with weight 1.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                   int k, int ns, int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;                      // whole waves exit together
  const float* row = logits + t * E;
  float v[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -__builtin_inff();
  }
  uint32_t taken = 0;                      // bit i: element i of this lane already selected
  float sel_val[16];
  int sel_id[16];
  for (int j = 0; j < k; ++j) {
    // best untaken element of this lane (ids ascend with i, so '>' keeps the lower id)
    float bv = -__builtin_inff();
    int bid = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && (v[i] > bv || bid == 0x7FFFFFFF)) {
        bv = v[i];
        bid = e;
      }
    }
    // wave arg-max with ties to the lower id
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oid = __shfl_xor(bid, o, 64);
      if (ov > bv || (ov == bv && oid < bid)) {
        bv = ov;
        bid = oid;
      }
    }
    sel_val[j] = bv;
    sel_id[j] = bid;
    if ((bid & 63) == lane) taken |= 1u << (bid >> 6);
  }
  if (lane == 0) {
    float e[16];
    float total = 0.0f;
    for (int j = 0; j < k; ++j) {
      e[j] = exp_f32(sel_val[j] - sel_val[0]);
      total = j == 0 ? e[0] : total + e[j];
    }
    const int kk = k + ns;
    for (int j = 0; j < k; ++j) {
      ids[t * kk + j] = sel_id[j];
      w[t * kk + j] = e[j] / total;
    }
    for (int j = 0; j < ns; ++j) {
      ids[t * kk + k + j] = E + j;
      w[t * kk + k + j] = 1.0f;
    }
  }
}

// One block per expert e.  Pass 1 counts the flat (token, slot) entries with
// an id below e (that count is e's offset) and equal to e.  Pass 2 gives each
// entry of e its rank among e's entries in flat order: every wave owns one
// contiguous range of flat indices, ranks inside the wave come from a ballot,
// and the ranges are offset by the counts of the waves before.  No atomics, so
// the permutation is the same on every run.  Both passes read a wave's range
// kPermBatch x 64 ids at a time, all loads issued before the first is used,
// so that a pass costs one memory round trip per batch instead of one per 64
// ids; pass 2 still takes the batch's 64-id chunks in flat order.
constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;
constexpr int kPermBatch = 8;

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ ids, int64_t R,
                                                               int k, int E, int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_ids,
                                                               int32_t* __restrict__ inv) {
  __shared__ int32_t wave_eq[kPermWaves];
  __shared__ int32_t wave_lt[kPermWaves];
  const int e = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t per_wave = (R + kPermWaves - 1) / kPermWaves;
  const int64_t lo = wv * per_wave;
  const int64_t hi = lo + per_wave < R ? lo + per_wave : R;
  int32_t n_lt = 0, n_eq = 0;
  for (int64_t b = lo; b < hi; b += 64 * kPermBatch) {
    int32_t v[kPermBatch];
#pragma unroll
    for (int u = 0; u < kPermBatch; ++u) {
      const int64_t f = b + 64 * u + lane;
      v[u] = f < hi ? ids[f] : INT32_MAX;
    }
#pragma unroll
    for (int u = 0; u < kPermBatch; ++u) {
      n_lt += v[u] < e;
      n_eq += v[u] == e;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    n_lt += __shfl_xor(n_lt, o, 64);
    n_eq += __shfl_xor(n_eq, o, 64);
  }
  if (lane == 0) {
    wave_lt[wv] = n_lt;
    wave_eq[wv] = n_eq;
  }
  __syncthreads();
  int32_t base = 0, total_lt = 0, total_eq = 0;
  for (int i = 0; i < kPermWaves; ++i) {
    if (i < wv) base += wave_eq[i];
    total_lt += wave_lt[i];
    total_eq += wave_eq[i];
  }
  if (threadIdx.x == 0) {
    offsets[e] = total_lt;
    if (e == E - 1) offsets[E] = total_lt + total_eq;
  }
  if (total_eq == 0) return;
  int32_t pos = total_lt + base;
  for (int64_t b = lo; b < hi; b += 64 * kPermBatch) {
    int32_t v[kPermBatch];
#pragma unroll
    for (int u = 0; u < kPermBatch; ++u) {
      const int64_t f = b + 64 * u + lane;
      v[u] = f < hi ? ids[f] : INT32_MAX;
    }
#pragma unroll
    for (int u = 0; u < kPermBatch; ++u) {
      const int64_t f = b + 64 * u + lane;
      const bool mine = v[u] == e;     // INT32_MAX (past the range) is never an expert id
      const uint64_t mask = __ballot(mine);
      const uint64_t below = lane ? (mask & ((~0ull) >> (64 - lane))) : 0ull;
      if (mine) {
        const int32_t p = pos + (int32_t)__popcll(below);
        sorted_ids[p] = (int32_t)(f / k);
        inv[f] = p;
      }
      pos += (int32_t)__popcll(mask);
    }
  }
}

__global__ void zero_offsets_kernel(int32_t* offsets, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) offsets[i] = 0;
}

hipError_t launch_route_permute(const float* logits, int64_t T, int E, int k, int ns, int32_t* ids, float* w,
                                int32_t* offsets, int32_t* sorted_ids, int32_t* inv, hipStream_t s) {
  // the shared experts are groups E .. E+ns-1 of the permutation, each
  // token's slots k .. k+ns-1
  const int G = E + ns, kk = k + ns;
  if (T == 0) {
    hipLaunchKernelGGL(zero_offsets_kernel, dim3(1), dim3(256), 0, s, offsets, G + 1);
    return hipGetLastError();
  }
  const int64_t blocks = (T + 3) / 4;      // 4 tokens (waves) per block
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)blocks), dim3(256), 0, s, logits, T, E, k, ns, ids, w);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(permute_kernel, dim3((unsigned)G), dim3(kPermThreads), 0, s, ids, T * kk, kk, G,
                     offsets, sorted_ids, inv);
  return hipGetLastError();
}

}  // namespace nvfp4
