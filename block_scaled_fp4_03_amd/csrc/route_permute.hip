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

// The stable group-by-expert permutation as a counting sort.  The flat
// (token, slot) entries are cut into nb contiguous chunks, one block each;
// inside a block, wave w owns the w-th contiguous part of the chunk.
//  * count (nb > 1): block b counts its chunk per group into row b of a
//    scratch table (nb x G ints; the sorted_ids array serves, nb * G <= R).
//  * scan: thread e turns column e into group e's offset (the exclusive sum
//    of all groups' totals, a block scan) and each block's first position for
//    e (the offset plus e's entries in the chunks before).
//  * rank: each wave counts its part per group (local atomic adds: counts
//    only, their order does not matter); thread e turns the block's first
//    position for e into each wave's; then each wave walks its part in flat
//    order, 64 entries at a time: the lanes holding the same id find each
//    other with one ballot per id bit, an entry's position is its wave's
//    running position for that id plus the number of equal ids in lower
//    lanes, and the highest such lane advances the running position.
//  * scatter (nb > 1): sorted_ids[inv[f]] = token of f, once the scratch
//    table is no longer read.
// With nb == 1 one block does the scan and the rank and writes every output.
// Every position follows from the flat order alone, so the permutation is the
// same on every run; the work is O(R + G * nb).
constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;
constexpr int kPermBatch = 8;
constexpr int kPermMaxGroups = 1024;
constexpr int64_t kPermChunk = 4096;          // entries per block when nb > 1

// wave-level inclusive scan of x, then the block-level exclusive prefix of
// the block's threads in order; returns the exclusive prefix of this thread
// and writes the block total to *sum_out (all threads)
__device__ __forceinline__ int32_t block_excl_scan(int32_t x, int32_t* wave_sum, int32_t& block_total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int32_t incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wave_sum[wv] = incl;
  __syncthreads();
  int32_t before = 0;
  block_total = 0;
  for (int w = 0; w < kPermWaves; ++w) {
    if (w < wv) before += wave_sum[w];
    block_total += wave_sum[w];
  }
  return before + incl - x;
}

__global__ __launch_bounds__(kPermThreads) void perm_count_kernel(const int32_t* __restrict__ ids, int64_t R, int G,
                                                                  int32_t* __restrict__ table) {
  __shared__ int32_t cnt[kPermMaxGroups];
  for (int e = threadIdx.x; e < G; e += kPermThreads) cnt[e] = 0;
  __syncthreads();
  const int64_t lo = (int64_t)blockIdx.x * kPermChunk;
  const int64_t hi = lo + kPermChunk < R ? lo + kPermChunk : R;
  for (int64_t f = lo + threadIdx.x; f < hi; f += kPermThreads) {
    const int32_t v = ids[f];
    if (v >= 0 && v < G) atomicAdd(&cnt[v], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G; e += kPermThreads) table[(int64_t)blockIdx.x * G + e] = cnt[e];
}

__global__ __launch_bounds__(kPermThreads) void perm_scan_kernel(int nb, int G, int32_t* __restrict__ table,
                                                                 int32_t* __restrict__ offsets) {
  __shared__ int32_t wave_sum[kPermWaves];
  const int e = threadIdx.x;
  int32_t total = 0;
  if (e < G)
    for (int b = 0; b < nb; ++b) total += table[(int64_t)b * G + e];
  int32_t all;
  const int32_t off = block_excl_scan(total, wave_sum, all);
  if (e < G) {
    offsets[e] = off;
    int32_t run = off;
    for (int b = 0; b < nb; ++b) {
      const int32_t c = table[(int64_t)b * G + e];
      table[(int64_t)b * G + e] = run;
      run += c;
    }
  }
  if (e == 0) offsets[G] = all;
}

// rank: block b takes chunk b (nb > 1: of kPermChunk entries, its first
// positions in row b of `table`; nb == 1: every entry, first positions from
// its own scan, offsets and sorted_ids written here)
__global__ __launch_bounds__(kPermThreads) void perm_rank_kernel(const int32_t* __restrict__ ids, int64_t R, int k,
                                                                 int G, int nb, const int32_t* table,
                                                                 int32_t* __restrict__ offsets, int32_t* sorted_ids,
                                                                 int32_t* __restrict__ inv) {
  __shared__ int32_t cnt[kPermWaves * kPermMaxGroups];   // [wave][group], row stride G
  __shared__ int32_t wave_sum[kPermWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  for (int i = tid; i < kPermWaves * G; i += kPermThreads) cnt[i] = 0;
  __syncthreads();
  const int64_t c_lo = nb > 1 ? (int64_t)blockIdx.x * kPermChunk : 0;
  const int64_t c_hi = nb > 1 ? (c_lo + kPermChunk < R ? c_lo + kPermChunk : R) : R;
  const int64_t per_wave = (c_hi - c_lo + kPermWaves - 1) / kPermWaves;
  const int64_t lo = c_lo + wv * per_wave < c_hi ? c_lo + wv * per_wave : c_hi;
  const int64_t hi = lo + per_wave < c_hi ? lo + per_wave : c_hi;
  for (int64_t b = lo; b < hi; b += 64 * kPermBatch) {
    int32_t v[kPermBatch];
#pragma unroll
    for (int u = 0; u < kPermBatch; ++u) {
      const int64_t f = b + 64 * u + lane;
      v[u] = f < hi ? ids[f] : -1;
    }
#pragma unroll
    for (int u = 0; u < kPermBatch; ++u)
      if (v[u] >= 0 && v[u] < G) atomicAdd(&cnt[wv * G + v[u]], 1);
  }
  __syncthreads();
  // the block's first position for group e: from the table, or (one block)
  // the exclusive scan of the totals, which is also e's offset
  const int e = tid;
  int32_t first = 0;
  if (nb > 1) {
    if (e < G) first = table[(int64_t)blockIdx.x * G + e];
  } else {
    int32_t total = 0;
    if (e < G)
      for (int w = 0; w < kPermWaves; ++w) total += cnt[w * G + e];
    int32_t all;
    first = block_excl_scan(total, wave_sum, all);
    if (e < G) offsets[e] = first;
    if (e == 0) offsets[G] = all;
  }
  if (e < G) {
    int32_t run = first;
    for (int w = 0; w < kPermWaves; ++w) {
      const int32_t c = cnt[w * G + e];
      cnt[w * G + e] = run;
      run += c;
    }
  }
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < G) ++nbits;
  const uint64_t lower = lane ? ((~0ull) >> (64 - lane)) : 0ull;
  for (int64_t b = lo; b < hi; b += 64 * kPermBatch) {
    int32_t v[kPermBatch];
#pragma unroll
    for (int u = 0; u < kPermBatch; ++u) {
      const int64_t f = b + 64 * u + lane;
      v[u] = f < hi ? ids[f] : -1;
    }
#pragma unroll
    for (int u = 0; u < kPermBatch; ++u) {
      if (b + 64 * u >= hi) break;       // (uniform) the rest of the batch is past the part
      const int64_t f = b + 64 * u + lane;
      const bool valid = v[u] >= 0 && v[u] < G;
      uint64_t peers = __ballot(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool set = (v[u] >> bit) & 1;
        const uint64_t m = __ballot(set);
        peers &= set ? m : ~m;
      }
      if (valid) {
        const int32_t p = cnt[wv * G + v[u]] + (int32_t)__popcll(peers & lower);
        if (nb == 1) sorted_ids[p] = (int32_t)(f / k);
        inv[f] = p;
      }
      // one wave's local-memory operations complete in program order: every
      // lane has read its running position before the highest lane of each
      // id advances it
      if (valid && (peers >> lane) == 1ull) cnt[wv * G + v[u]] += (int32_t)__popcll(peers);
    }
  }
}

__global__ __launch_bounds__(256) void perm_scatter_kernel(const int32_t* __restrict__ inv, int64_t R, int k,
                                                           int32_t* __restrict__ sorted_ids) {
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (f < R) sorted_ids[inv[f]] = (int32_t)(f / k);
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
  if (G > kPermMaxGroups) return hipErrorInvalidValue;   // (the C ABI admits at most 1024 groups)
  const int64_t R = T * kk;
  // blocks of kPermChunk entries, as long as their table fits sorted_ids
  int64_t nb = (R + kPermChunk - 1) / kPermChunk;
  if (nb * G > R) nb = 1;
  if (nb == 1) {
    hipLaunchKernelGGL(perm_rank_kernel, dim3(1), dim3(kPermThreads), 0, s, ids, R, kk, G, 1,
                       (const int32_t*)nullptr, offsets, sorted_ids, inv);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(perm_count_kernel, dim3((unsigned)nb), dim3(kPermThreads), 0, s, ids, R, G, sorted_ids);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(kPermThreads), 0, s, (int)nb, G, sorted_ids, offsets);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(perm_rank_kernel, dim3((unsigned)nb), dim3(kPermThreads), 0, s, ids, R, kk, G, (int)nb,
                     (const int32_t*)sorted_ids, offsets, sorted_ids, inv);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(perm_scatter_kernel, dim3((unsigned)((R + 255) / 256)), dim3(256), 0, s, inv, R, kk,
                     sorted_ids);
  return hipGetLastError();
}

}  // namespace nvfp4
