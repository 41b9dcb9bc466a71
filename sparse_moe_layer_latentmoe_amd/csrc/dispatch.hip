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
//   scatter one wave per block again: row p of slot (t, k) = offsets[e] +
//           prefix[block][e] + number of earlier tokens of the block with e.
//
// For small token counts the three phases run in one work-group.
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
    for (int k0 = 0; k0 < K; k0 += 8) {
      int ex[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ex[i] = k0 + i < K ? idx[(size_t)t * K + k0 + i] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (k0 + i < K) atomicOr(&mask[ex[i]], 1ull << lane);
    }
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
    // blockcnt[b][e] <- rows of e in blocks before b; sixteen blocks' loads
    // in flight at a time
    for (int b0 = 0; b0 < nblocks; b0 += 16) {
      int c[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = b0 + i < nblocks ? blockcnt[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (b0 + i < nblocks) {
          blockcnt[(size_t)(b0 + i) * E + e] = n;
          n += c[i];
        }
    }
  }
  const int off = block_exclusive_scan(e < E ? n : 0, scratch, &tot_rows);
  const int nt = (n + tile_m - 1) / tile_m;
  const int toff = block_exclusive_scan(e < E ? nt : 0, scratch, &tot_tiles);
  if (e < E) {
    counts[e] = n;
    offsets[e] = off;
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
                                                              const int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ rows_tok,
                                                              int32_t* __restrict__ inv) {
  __shared__ unsigned long long mask[1024];
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  for (int e = lane; e < E; e += 64) mask[e] = 0ull;
  __syncthreads();
  const int t = b * 64 + lane;
  if (t < T)
    for (int k0 = 0; k0 < K; k0 += 8) {
      int ex[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ex[i] = k0 + i < K ? idx[(size_t)t * K + k0 + i] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (k0 + i < K) atomicOr(&mask[ex[i]], 1ull << lane);
    }
  __syncthreads();
  if (t < T) {
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    // row = expert offset + rows of e in earlier blocks + earlier tokens of
    // this block with e; eight slots' loads in flight at a time
    for (int k0 = 0; k0 < K; k0 += 8) {
      int ex[8], p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ex[i] = k0 + i < K ? idx[(size_t)t * K + k0 + i] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        p[i] = offsets[ex[i]] + blockbase[(size_t)b * E + ex[i]] + __popcll(mask[ex[i]] & below);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (k0 + i < K) {
          rows_tok[p[i]] = t;
          inv[(size_t)t * K + k0 + i] = p[i];
        }
    }
  }
}

// The same three phases in one work-group, for token counts whose per-block
// masks and bases fit in LDS (decode and speculative-verify batches): one
// launch instead of three.  Wave w handles token blocks w, w + 16, ...;
// thread e handles expert e.  Rows and tiles come out exactly as above.
__global__ __launch_bounds__(1024) void dispatch_fused_kernel(
    const int32_t* __restrict__ idx, int T, int K, int E, int nb, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ rows_tok, int32_t* __restrict__ inv,
    Tile* __restrict__ tiles, int32_t* __restrict__ ntiles, int tile_m) {
  extern __shared__ unsigned long long dmask[];  // [nb][E] masks, then [nb][E] int bases
  int* base = reinterpret_cast<int*>(dmask + (size_t)nb * E);
  __shared__ int scratch[32];
  __shared__ int tot_rows, tot_tiles;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i < nb * E; i += 1024) dmask[i] = 0ull;
  __syncthreads();
  for (int b = wv; b < nb; b += 16) {
    const int t = b * 64 + lane;
    if (t < T)
      for (int k = 0; k < K; ++k)
        atomicOr(&dmask[(size_t)b * E + idx[(size_t)t * K + k]], 1ull << lane);
  }
  __syncthreads();
  const int e = tid;
  int n = 0;
  if (e < E)
    for (int b = 0; b < nb; ++b) {
      base[b * E + e] = n;
      n += __popcll(dmask[(size_t)b * E + e]);
    }
  const int off = block_exclusive_scan(e < E ? n : 0, scratch, &tot_rows);
  const int nt = (n + tile_m - 1) / tile_m;
  const int toff = block_exclusive_scan(e < E ? nt : 0, scratch, &tot_tiles);
  if (e < E) {
    counts[e] = n;
    offsets[e] = off;
    for (int b = 0; b < nb; ++b) base[b * E + e] += off;
    for (int i = 0; i < nt; ++i) {
      Tile tl;
      tl.expert = e;
      tl.row0 = off + i * tile_m;
      tl.nrows = min(tile_m, n - i * tile_m);
      tl.first = toff;
      tl.count = nt;
      tl.pad0 = tl.pad1 = tl.pad2 = 0;
      tiles[toff + i] = tl;
    }
  }
  if (e == 0) {
    offsets[E] = tot_rows;
    *ntiles = tot_tiles;
  }
  __syncthreads();
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int b = wv; b < nb; b += 16) {
    const int t = b * 64 + lane;
    if (t < T)
      for (int k = 0; k < K; ++k) {
        const int ex = idx[(size_t)t * K + k];
        const int p = base[b * E + ex] + __popcll(dmask[(size_t)b * E + ex] & below);
        rows_tok[p] = t;
        inv[(size_t)t * K + k] = p;
      }
  }
}

// r[t][c..c+7] = sum_k w[t][k] * O[inv[t][k]][c..c+7], k ascending (= ascending
// expert id), fp32; stored bf16 (the fc2_latent input) and optionally fp32.
// Work-group (t, chunk): one token, 2048 columns (8 per thread).  The token's
// K row indices and weights are staged in LDS once, then each thread issues
// its row loads eight at a time, so the K loads overlap instead of forming a
// chain of dependent memory round trips.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ o,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int T, int K,
                                                      int R, uint16_t* __restrict__ r16,
                                                      float* __restrict__ r32) {
  __shared__ int32_t sp[64];
  __shared__ float sw[64];
  const int t = blockIdx.x;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (threadIdx.x < K) {
    sp[threadIdx.x] = inv[(size_t)t * K + threadIdx.x];
    sw[threadIdx.x] = w[(size_t)t * K + threadIdx.x];
  }
  __syncthreads();
  if (c >= R) return;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  constexpr int B = 8;
  for (int k0 = 0; k0 < K; k0 += B) {
    bf16x8 v[B];
#pragma unroll
    for (int b = 0; b < B; ++b)
      if (k0 + b < K) v[b] = load8(o + (size_t)sp[k0 + b] * R + c);
#pragma unroll
    for (int b = 0; b < B; ++b)
      if (k0 + b < K) {
        const float wk = sw[k0 + b];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += wk * static_cast<float>(v[b][i]);
      }
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
  const size_t fused_lds = (size_t)nb * E * (sizeof(unsigned long long) + sizeof(int));
  if (E <= 1024 && fused_lds <= 65536) {
    dispatch_fused_kernel<<<1, 1024, fused_lds, s>>>(idx, T, K, E, nb, counts, offsets, rows_tok,
                                                     inv, tiles, ntiles, tile_m);
    return hipGetLastError();
  }
  dispatch_hist_kernel<<<nb, 64, 0, s>>>(idx, T, K, E, blockcnt);
  dispatch_scan_kernel<<<1, 1024, 0, s>>>(blockcnt, nb, E, counts, offsets, tiles, ntiles, tile_m);
  dispatch_scatter_kernel<<<nb, 64, 0, s>>>(idx, T, K, E, blockcnt, offsets, rows_tok, inv);
  return hipGetLastError();
}

hipError_t combine(const uint16_t* o, const int32_t* inv, const float* w, int T, int K, int R,
                   uint16_t* r16, float* r32, hipStream_t s) {
  if (T <= 0 || R <= 0) return hipSuccess;
  const dim3 grid(T, (R + 2047) / 2048);
  combine_kernel<<<grid, 256, 0, s>>>(o, inv, w, T, K, R, r16, r32);
  return hipGetLastError();
}

}  // namespace lmoe
