// Token -> expert grouping and the weighted combine.
//
// The page's reference loop (page "Nemotron 3 Ultra 架构深度拆解报告", CH5
// §5.6 Step 6) builds a one-hot expert mask, visits only the experts that
// received tokens, gathers their token rows, and scatter-adds weighted
// outputs with index_add_.  Here the same grouping is a stable counting
// sort of the T*K (token, expert) slots by expert, computed on the device
// with no host round trip:
//
//   hist    one wave per 64-token block: per expert a 64-bit LDS mask of the
//           block's tokens that chose it; block histogram = popcount.
//   scan    one work-group: per expert, exclusive prefix over blocks, the
//           expert totals (counts), their exclusive prefix (offsets), and the
//           work-tile list over non-empty experts (empty experts get none).
//   scatter one wave per block again: row p of slot (t, k) =
//           base[block][e] + number of earlier tokens of the block with e.
//
// Rows of one expert are therefore in token order, so everything downstream
// is deterministic.  The combine (replacing index_add_) gathers each token's
// K expert rows in ascending expert id, multiplies by the routing weight and
// adds in fp32.
#include "kernels.h"
#include "lmoe_device.h"

namespace lmoe {

__global__ __launch_bounds__(64) void dispatch_hist_kernel(const int32_t* __restrict__ idx, int T,
                                                           int K, int E,
                                                           int32_t* __restrict__ blockcnt) {
  __shared__ unsigned long long mask[1024];
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  for (int e = lane; e < E; e += 64) mask[e] = 0ull;
  __syncthreads();
  const int t = b * 64 + lane;
  if (t < T)
    for (int k = 0; k < K; ++k) atomicOr(&mask[idx[(size_t)t * K + k]], 1ull << lane);
  __syncthreads();
  for (int e = lane; e < E; e += 64) blockcnt[(size_t)b * E + e] = __popcll(mask[e]);
}

// Exclusive scan of v over the first n entries of a 1024-thread block.
__device__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off, 64);
    if (lane >= off) inc += o;
  }
  if (lane == 63) scratch[wv] = inc;
  __syncthreads();
  if (wv == 0) {
    int x = lane < 16 ? scratch[lane] : 0;
    int xi = x;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int o = __shfl_up(xi, off, 64);
      if (lane >= off) xi += o;
    }
    if (lane < 16) scratch[16 + lane] = xi - x;
    if (lane == 15) *total = xi;
  }
  __syncthreads();
  const int r = scratch[16 + wv] + inc - v;
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(1024) void dispatch_scan_kernel(int32_t* __restrict__ blockcnt,
                                                             int nblocks, int E,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             Tile* __restrict__ tiles,
                                                             int32_t* __restrict__ ntiles,
                                                             int tile_m) {
  __shared__ int scratch[32];
  __shared__ int tot_rows, tot_tiles;
  const int e = threadIdx.x;
  int n = 0;
  if (e < E) {
    for (int b = 0; b < nblocks; ++b) {
      const int c = blockcnt[(size_t)b * E + e];
      blockcnt[(size_t)b * E + e] = n;
      n += c;
    }
  }
  const int off = block_exclusive_scan(e < E ? n : 0, scratch, &tot_rows);
  const int nt = (n + tile_m - 1) / tile_m;
  const int toff = block_exclusive_scan(e < E ? nt : 0, scratch, &tot_tiles);
  if (e < E) {
    counts[e] = n;
    offsets[e] = off;
    for (int b = 0; b < nblocks; ++b) blockcnt[(size_t)b * E + e] += off;
    for (int i = 0; i < nt; ++i) {
      Tile t;
      t.expert = e;
      t.row0 = off + i * tile_m;
      t.nrows = min(tile_m, n - i * tile_m);
      t.first = toff;
      t.count = nt;
      t.pad0 = t.pad1 = t.pad2 = 0;
      tiles[toff + i] = t;
    }
  }
  if (e == 0) {
    offsets[E] = tot_rows;
    *ntiles = tot_tiles;
  }
}

__global__ __launch_bounds__(64) void dispatch_scatter_kernel(const int32_t* __restrict__ idx,
                                                              int T, int K, int E,
                                                              const int32_t* __restrict__ blockbase,
                                                              int32_t* __restrict__ rows_tok,
                                                              int32_t* __restrict__ inv) {
  __shared__ unsigned long long mask[1024];
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  for (int e = lane; e < E; e += 64) mask[e] = 0ull;
  __syncthreads();
  const int t = b * 64 + lane;
  if (t < T)
    for (int k = 0; k < K; ++k) atomicOr(&mask[idx[(size_t)t * K + k]], 1ull << lane);
  __syncthreads();
  if (t < T) {
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int k = 0; k < K; ++k) {
      const int e = idx[(size_t)t * K + k];
      const int p = blockbase[(size_t)b * E + e] + __popcll(mask[e] & below);
      rows_tok[p] = t;
      inv[(size_t)t * K + k] = p;
    }
  }
}

// r[t][c..c+7] = sum_k w[t][k] * O[inv[t][k]][c..c+7], k ascending (= ascending
// expert id), fp32; stored bf16 (the fc2_latent input) and optionally fp32.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ o,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int T, int K,
                                                      int R, uint16_t* __restrict__ r16,
                                                      float* __restrict__ r32) {
  const int cpr = R / 8;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)T * cpr) return;
  const int t = gid / cpr;
  const int c = (gid % cpr) * 8;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int k = 0; k < K; ++k) {
    const int p = inv[(size_t)t * K + k];
    const float wk = w[(size_t)t * K + k];
    const bf16x8 v = load8(o + (size_t)p * R + c);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += wk * static_cast<float>(v[i]);
  }
  u16x4 lo, hi;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo[i] = f32_to_bf16(acc[i]);
    hi[i] = f32_to_bf16(acc[4 + i]);
  }
  *reinterpret_cast<u16x4*>(r16 + (size_t)t * R + c) = lo;
  *reinterpret_cast<u16x4*>(r16 + (size_t)t * R + c + 4) = hi;
  if (r32) {
    *reinterpret_cast<f32x4*>(r32 + (size_t)t * R + c) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(r32 + (size_t)t * R + c + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

hipError_t dispatch(const int32_t* idx, int T, int K, int E, int32_t* blockcnt, int32_t* counts,
                    int32_t* offsets, int32_t* rows_tok, int32_t* inv, Tile* tiles,
                    int32_t* ntiles, int tile_m, hipStream_t s) {
  const int nb = (T + 63) / 64;
  dispatch_hist_kernel<<<nb, 64, 0, s>>>(idx, T, K, E, blockcnt);
  dispatch_scan_kernel<<<1, 1024, 0, s>>>(blockcnt, nb, E, counts, offsets, tiles, ntiles, tile_m);
  dispatch_scatter_kernel<<<nb, 64, 0, s>>>(idx, T, K, E, blockcnt, rows_tok, inv);
  return hipGetLastError();
}

hipError_t combine(const uint16_t* o, const int32_t* inv, const float* w, int T, int K, int R,
                   uint16_t* r16, float* r32, hipStream_t s) {
  const long n = (long)T * (R / 8);
  if (n <= 0) return hipSuccess;
  combine_kernel<<<(n + 255) / 256, 256, 0, s>>>(o, inv, w, T, K, R, r16, r32);
  return hipGetLastError();
}

}  // namespace lmoe
