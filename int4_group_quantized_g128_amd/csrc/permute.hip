// A5 group-by-expert permutation of the routed slots and the row-tile list.
//
// Page "MoE推理优化实战：4bit存储+INT8计算的W4A8路线解析" §1: dispatching tokens to
// experts and combining the results are costs of their own; this is the dispatch step.
//
// One workgroup of up to 16 waves.  Wave w owns a contiguous range of slots.
//   pass 1: per-wave expert counts in LDS;
//   pass 2: counts, offsets (exclusive scan) and each wave's base per expert;
//   pass 3: each wave walks its range 64 slots at a time in slot order; lanes with the
//           same expert find their rank with ballots, so the scatter is stable.
#include "common.h"
#include "internal.h"

namespace q4 {

constexpr int kPermThreads = 1024;

// Exclusive scan of n ints in LDS (in place); returns the total.  All threads call.
__device__ int32_t block_exclusive_scan(int32_t* data, int n, int32_t* wave_tot) {
  const int tid = threadIdx.x;
  const int per = (n + kPermThreads - 1) / kPermThreads;
  const int beg = tid * per, end = min(n, beg + per);
  int32_t local = 0;
  for (int i = beg; i < end; ++i) local += data[i];
  // inclusive scan of 'local' across the block
  const int lane = tid & 63, wid = tid >> 6;
  int32_t v = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) wave_tot[wid] = v;
  __syncthreads();
  if (wid == 0) {   // exclusive scan of the wave totals by wave 0 (each lane reads, then writes, its own)
    constexpr int nw = kPermThreads / 64;
    const int32_t x = lane < nw ? wave_tot[lane] : 0;
    int32_t incl = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    if (lane < nw) wave_tot[lane] = incl - x;
    if (lane == nw - 1) wave_tot[nw] = incl;
  }
  __syncthreads();
  int32_t run = v - local + wave_tot[wid];
  for (int i = beg; i < end; ++i) {
    const int32_t x = data[i];
    data[i] = run;
    run += x;
  }
  const int32_t total = wave_tot[kPermThreads / 64];
  __syncthreads();
  return total;
}

// Weight format of expert x for the tile order: 0 = 4-bit with one scale entry per tile,
// 1 = two entries (groups of 64), 2 = four (groups of 32), 3 = 8-bit.
__device__ __forceinline__ int tile_format(const uint8_t* ebits, const uint8_t* egroups, int x) {
  if (ebits && ebits[x] == 8) return 3;
  if (egroups) {
    const int sg = sg_of_code(egroups[x]);
    return sg == 4 ? 2 : sg == 2 ? 1 : 0;
  }
  return 0;
}

__global__ void __launch_bounds__(kPermThreads) k_permute(const int32_t* __restrict__ ids, int64_t t, int32_t k,
                                                          int32_t e, int shared, int nwaves,
                                                          int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                                          TileDesc* __restrict__ tiles, int32_t* __restrict__ num_tiles,
                                                          int tile_rows, const uint8_t* __restrict__ ebits,
                                                          const uint8_t* __restrict__ egroups,
                                                          int32_t* __restrict__ fmt_tiles) {
  extern __shared__ int32_t lds[];
  __shared__ int32_t wave_tot[kPermThreads / 64 + 1];
  const int ee = e + shared;            // experts incl. the shared one
  const int S = k + shared;             // slots per token
  const int64_t P = t * S;
  int32_t* cnt = lds;                   // [nwaves][ee]
  int32_t* tot = lds + nwaves * ee;     // [ee + 1]
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  for (int i = tid; i < nwaves * ee + ee + 1; i += kPermThreads) lds[i] = 0;
  __syncthreads();
  const int64_t per = (P + nwaves - 1) / nwaves;
  const int64_t beg = std::min<int64_t>(P, int64_t(wid) * per), end = std::min<int64_t>(P, beg + per);
  auto expert_of = [&](int64_t s) -> int {
    const int64_t tok = s / S;
    const int j = int(s - tok * S);
    if (j >= k) return e;               // the shared expert
    int x = ids[tok * k + j];
    return min(max(x, 0), e - 1);       // out-of-range ids are clamped
  };
  // pass 1 (the experts of a lane's first kKeep slots stay in registers for pass 3)
  constexpr int kKeep = 4;
  int kept[kKeep];
  if (wid < nwaves) {
    int i = 0;
    for (int64_t s = beg + lane; s < end; s += 64, ++i) {
      const int x = expert_of(s);
#pragma unroll
      for (int j = 0; j < kKeep; ++j)
        if (i == j) kept[j] = x;
      atomicAdd(&cnt[wid * ee + x], 1);
    }
  }
  __syncthreads();
  // pass 2: totals, offsets, per-wave bases
  for (int x = tid; x < ee; x += kPermThreads) {
    int32_t run = 0;
    for (int w = 0; w < nwaves; ++w) run += cnt[w * ee + x];
    tot[x] = run;
  }
  __syncthreads();
  // LDS after cnt [nwaves][ee] and tot [ee + 1]: counts, offsets, tiles per expert,
  // first tile of each expert ([ee] each)
  int32_t* cntl = lds + nwaves * ee + ee + 1;
  int32_t* offl = cntl + ee;
  int32_t* ntl = offl + ee;
  int32_t* first = ntl + ee;
  for (int x = tid; x < ee; x += kPermThreads) {
    counts[x] = tot[x];
    cntl[x] = tot[x];
  }
  __syncthreads();
  const int32_t total = block_exclusive_scan(tot, ee, wave_tot);
  for (int x = tid; x < ee; x += kPermThreads) {
    offsets[x] = tot[x];
    offl[x] = tot[x];
    int32_t run = tot[x];
    for (int w = 0; w < nwaves; ++w) {
      const int32_t c = cnt[w * ee + x];
      cnt[w * ee + x] = run;
      run += c;
    }
  }
  if (tid == 0) offsets[ee] = total;
  __syncthreads();
  // pass 3: stable scatter
  int nbits = 1;
  while ((1 << nbits) <= ee) ++nbits;
  if (wid < nwaves) {
    int i = 0;
    for (int64_t s0 = beg; s0 < end; s0 += 64, ++i) {
      const int64_t s = s0 + lane;
      const bool valid = s < end;
      int ex = 0;
      if (i < kKeep) {
#pragma unroll
        for (int j = 0; j < kKeep; ++j)
          if (i == j && valid) ex = kept[j];
      } else if (valid) {
        ex = expert_of(s);
      }
      unsigned long long peers = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const unsigned long long m = __ballot((ex >> b) & 1);
        peers &= ((ex >> b) & 1) ? m : ~m;
      }
      const unsigned long long below = peers & ((1ull << lane) - 1ull);
      const int rank = __popcll(below);
      int32_t pos = 0;
      if (valid) pos = cnt[wid * ee + ex] + rank;
      // make sure every lane has read the base before the leader advances it
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      if (valid) {
        perm[pos] = int32_t(s);
        inv[s] = pos;
        if (below == 0) cnt[wid * ee + ex] += __popcll(peers);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
  }
  // tile list: ceil(count / tile_rows) tiles per expert, ordered by (weight format,
  // expert), so that a GEMM launch for one format walks one contiguous range of tiles;
  // fmt_tiles[f] .. fmt_tiles[f + 1] is format f's range
  if (tiles) {
    __syncthreads();
    for (int x = tid; x < ee; x += kPermThreads) ntl[x] = (cntl[x] + tile_rows - 1) / tile_rows;
    __syncthreads();
    int32_t base = 0;
    const int nfmt = (ebits || egroups) ? 4 : 1;   // one format unless the layer mixes them
    for (int f = 0; f < 4; ++f) {
      if (f >= nfmt) {
        if (fmt_tiles && tid == 0) fmt_tiles[f] = base;
        continue;
      }
      for (int x = tid; x < ee; x += kPermThreads) tot[x] = tile_format(ebits, egroups, x) == f ? ntl[x] : 0;
      __syncthreads();
      const int32_t nf = block_exclusive_scan(tot, ee, wave_tot);
      for (int x = tid; x < ee; x += kPermThreads)
        if (tile_format(ebits, egroups, x) == f) first[x] = base + tot[x];
      if (fmt_tiles && tid == 0) fmt_tiles[f] = base;
      base += nf;
      __syncthreads();
    }
    const int32_t ntiles = base;
    if (fmt_tiles && tid == 0) fmt_tiles[4] = ntiles;
    for (int x = tid; x < ee; x += kPermThreads) {
      const int32_t c = cntl[x], o = offl[x];
      int32_t ti = first[x];
      for (int32_t r = 0; r < c; r += tile_rows, ++ti) {
        TileDesc d;
        d.expert = x;
        d.row_start = o + r;
        d.rows = min(tile_rows, c - r);
        d.pad = 0;
        tiles[ti] = d;
      }
    }
    if (tid == 0) *num_tiles = ntiles;
  }
}

hipError_t launch_permute(const int32_t* ids, int64_t t, int32_t k, int32_t e, int shared, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* inv, TileDesc* tiles, int32_t* num_tiles,
                          int tile_rows, hipStream_t st, const uint8_t* ebits, const uint8_t* egroups,
                          int32_t* fmt_tiles) {
  const int ee = e + shared;
  const size_t budget = 96 * 1024;
  // one wave per 64 slots (at most 16, and as many as the LDS budget allows): the
  // per-expert loops of pass 2 walk every wave's counts, so idle waves only cost time
  const int64_t P = t * (k + shared);
  int nwaves = int(std::min<size_t>(16, (budget / sizeof(int32_t) - (5 * ee + 1)) / ee));
  nwaves = int(std::max<int64_t>(1, std::min<int64_t>(nwaves, (P + 63) / 64)));
  const size_t lds = (size_t(nwaves) * ee + 5 * ee + 1) * sizeof(int32_t);
  hipLaunchKernelGGL(k_permute, dim3(1), dim3(kPermThreads), lds, st, ids, t, k, e, shared, nwaves, counts,
                     offsets, perm, inv, tiles, num_tiles, tile_rows, ebits, egroups, fmt_tiles);
  return hipGetLastError();
}

}  // namespace q4
