// Token -> expert permutation: per-chunk histogram, one-workgroup scan, stable scatter.
//
// On one GPU, sending each token to its experts and merging the results back
// (breadlab.ai Beam inference post, section "Reading 23B active and 501B
// resident separately") is a grouping of the T*K (token, slot) pairs by expert.
// Pairs of an expert keep ascending pair order, with no value atomics, so the
// result is the same on every run:
//   hist:    one wave per chunk of 64 tokens builds, for every expert, a 64-bit
//            mask of the chunk's tokens routed to it (LDS atomic OR: the result
//            does not depend on the order), stores it and its popcount;
//   scan:    one workgroup turns the per-chunk counts into per-chunk bases and
//            the expert offsets, and (for the forward) lists the row tiles of
//            the grouped GEMMs;
//   scatter: a token's rank inside its chunk is the popcount of the mask bits
//            below it, so row = offset[e] + base[chunk][e] + rank.
// A token routes to each expert at most once, so one bit per token suffices.
#include "common.h"

namespace beam {

__global__ __launch_bounds__(64) void perm_hist_kernel(int T, int E, int K, const int32_t* __restrict__ ids,
                                                       uint64_t* __restrict__ masks, int32_t* __restrict__ counts) {
  __shared__ uint64_t m[kMaxExperts];
  const int c = blockIdx.x, lane = threadIdx.x;
  const int t = c * kChunk + lane;
  for (int e = lane; e < E; e += kWave) m[e] = 0ull;
  __syncthreads();
  if (t < T) {
    for (int k = 0; k < K; ++k) {
      const int e = ids[(size_t)t * K + k];
      if (e >= 0 && e < E) atomicOr(reinterpret_cast<unsigned long long*>(&m[e]), 1ull << lane);
    }
  }
  __syncthreads();
  for (int e = lane; e < E; e += kWave) {
    const uint64_t v = m[e];
    masks[(size_t)c * E + e] = v;
    counts[(size_t)c * E + e] = __popcll(v);
  }
}

// counts[c][e] -> exclusive prefix over chunks (in place); offsets = exclusive scan over experts.
__global__ __launch_bounds__(256) void perm_scan_kernel(int E, int nchunks, int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets, int tile_rows,
                                                        int32_t* __restrict__ tiles, int32_t* __restrict__ ntiles) {
  __shared__ int32_t tot[kMaxExperts];
  __shared__ int32_t ntl[kMaxExperts];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    int c = 0;
    for (; c + 16 <= nchunks; c += 16) {   // 16 loads in flight, then the running sum in chunk order
      int v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = counts[(size_t)(c + j) * E + e];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        counts[(size_t)(c + j) * E + e] = run;
        run += v[j];
      }
    }
    for (; c < nchunks; ++c) {
      const int v = counts[(size_t)c * E + e];
      counts[(size_t)c * E + e] = run;
      run += v;
    }
  }
  // exclusive prefix sums over the experts of the row counts and the tile counts: within each wave by
  // shuffles, then across the four waves through LDS (integer sums: any order gives the same result)
  const int mytot = (e < E) ? run : 0;
  const int myntl = (e < E && tile_rows > 0) ? (run + tile_rows - 1) / tile_rows : 0;
  const int lane = e % kWave, wv = e / kWave;
  int it = mytot, in = myntl;   // inclusive within the wave
#pragma unroll
  for (int d = 1; d < kWave; d *= 2) {
    const int ot = __shfl_up(it, d), on = __shfl_up(in, d);
    if (lane >= d) {
      it += ot;
      in += on;
    }
  }
  if (lane == kWave - 1) {
    tot[wv] = it;
    ntl[wv] = in;
  }
  __syncthreads();
  int bt = 0, bn = 0;   // the sums of the waves before this one
  for (int j = 0; j < wv; ++j) {
    bt += tot[j];
    bn += ntl[j];
  }
  const int nw = (int)blockDim.x / kWave;
  if (e == 0) {
    int at = 0, an = 0;
    for (int j = 0; j < nw; ++j) {
      at += tot[j];
      an += ntl[j];
    }
    offsets[E] = at;
    if (tile_rows > 0) ntiles[0] = an;
  }
  __syncthreads();
  tot[e] = bt + it - mytot;
  ntl[e] = bn + in - myntl;
  __syncthreads();
  if (e < E) {
    offsets[e] = tot[e];
    if (tile_rows > 0) {
      const int nt = (run + tile_rows - 1) / tile_rows;
      for (int i = 0; i < nt; ++i) {
        tiles[2 * (ntl[e] + i)] = e;
        tiles[2 * (ntl[e] + i) + 1] = i * tile_rows;
      }
    }
  }
}

__global__ __launch_bounds__(64) void perm_scatter_kernel(int T, int E, int K, const int32_t* __restrict__ ids,
                                                          const uint64_t* __restrict__ masks,
                                                          const int32_t* __restrict__ base,
                                                          const int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_pairs,
                                                          int32_t* __restrict__ pair_to_row) {
  const int c = blockIdx.x, lane = threadIdx.x;
  const int t = c * kChunk + lane;
  if (t >= T) return;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int k = 0; k < K; ++k) {
    const int p = t * K + k;
    const int e = ids[p];
    if (e < 0 || e >= E) continue;
    const size_t ce = (size_t)c * E + e;
    const int row = offsets[e] + base[ce] + __popcll(masks[ce] & below);
    sorted_pairs[row] = p;
    pair_to_row[p] = row;
  }
}

// Small T (at most kSmallChunks chunks): the three steps in one workgroup of
// 16 waves, wave w owning chunk w; masks, counts and bases stay in LDS.
constexpr int kSmallChunks = 16;

__global__ __launch_bounds__(1024) void perm_small_kernel(int T, int E, int K, const int32_t* __restrict__ ids,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_pairs,
                                                          int32_t* __restrict__ pair_to_row, int tile_rows,
                                                          int32_t* __restrict__ tiles,
                                                          int32_t* __restrict__ ntiles) {
  __shared__ uint64_t m[kSmallChunks][kMaxExperts];
  __shared__ int32_t base[kSmallChunks][kMaxExperts];
  __shared__ int32_t off[kMaxExperts];
  __shared__ int32_t toff[kMaxExperts];
  const int tid = threadIdx.x, c = tid / kWave, lane = tid % kWave;
  const int nchunks = (T + kChunk - 1) / kChunk;
  for (int e = lane; e < E; e += kWave) m[c][e] = 0ull;
  __syncthreads();
  const int t = c * kChunk + lane;
  if (c < nchunks && t < T) {
    for (int k = 0; k < K; ++k) {
      const int e = ids[(size_t)t * K + k];
      if (e >= 0 && e < E) atomicOr(reinterpret_cast<unsigned long long*>(&m[c][e]), 1ull << lane);
    }
  }
  __syncthreads();
  for (int e = lane; e < E; e += kWave) base[c][e] = c < nchunks ? __popcll(m[c][e]) : 0;
  __syncthreads();
  int run = 0;
  if (tid < E) {
    for (int q = 0; q < nchunks; ++q) {
      const int v = base[q][tid];
      base[q][tid] = run;
      run += v;
    }
    off[tid] = run;
    toff[tid] = tile_rows > 0 ? (run + tile_rows - 1) / tile_rows : 0;
  }
  __syncthreads();
  if (tid == 0) {   // E <= 256 sequential adds
    int acc = 0, tacc = 0;
    for (int i = 0; i < E; ++i) {
      const int v = off[i], n = toff[i];
      off[i] = acc; acc += v;
      toff[i] = tacc; tacc += n;
    }
    offsets[E] = acc;
    if (tile_rows > 0) ntiles[0] = tacc;
  }
  __syncthreads();
  if (tid < E) {
    offsets[tid] = off[tid];
    if (tile_rows > 0) {
      const int nt = (run + tile_rows - 1) / tile_rows;
      for (int i = 0; i < nt; ++i) {
        tiles[2 * (toff[tid] + i)] = tid;
        tiles[2 * (toff[tid] + i) + 1] = i * tile_rows;
      }
    }
  }
  if (c < nchunks && t < T) {
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int k = 0; k < K; ++k) {
      const int p = t * K + k;
      const int e = ids[p];
      if (e < 0 || e >= E) continue;
      const int row = off[e] + base[c][e] + __popcll(m[c][e] & below);
      sorted_pairs[row] = p;
      pair_to_row[p] = row;
    }
  }
}

hipError_t launch_permute(const Shape& s, int T, const int32_t* ids, int nchunks, uint64_t* masks,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_to_row,
                          int tile_rows, int32_t* tiles, int32_t* ntiles, hipStream_t stream) {
  if (nchunks <= kSmallChunks) {
    hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(1024), 0, stream, T, s.E, s.K, ids, offsets, sorted_pairs,
                       pair_to_row, tile_rows, tiles, ntiles);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(perm_hist_kernel, dim3(nchunks), dim3(64), 0, stream, T, s.E, s.K, ids, masks, counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(256), 0, stream, s.E, nchunks, counts, offsets, tile_rows,
                     tiles, ntiles);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(nchunks), dim3(64), 0, stream, T, s.E, s.K, ids, masks, counts,
                     offsets, sorted_pairs, pair_to_row);
  return hipGetLastError();
}

}  // namespace beam
