// Block-scaled FP4 (MXFP4) expert weights for the weight-streaming path.
//
// The pages train the experts in FP4 with E2M1 elements (page "Nemotron 3
// Ultra 架构深度拆解报告", CH8 §8.1: values 0, ±0.5, ±1, ±1.5, ±2, ±3, ±4,
// ±6) but give two different block layouts, so the layout is fixed here, as
// the one gfx950 decodes in hardware: blocks of 32 consecutive k of a weight
// row, each with a power-of-two scale 2^(byte - 127).  Decoding is exact
// into bf16, so the expert GEMMs run the bf16 MFMA on the exact dequantised
// weights (weights 4.25 bits, activations bf16).
//
//   quantise  one thread per block: X = 2^e with e = floor(log2 max|w|) - 2
//             (clipped to [-127, 127]; -127 for an all-zero block), each
//             element |w| / X rounded to the nearest E2M1 magnitude with
//             ties to the even code (zero mantissa bit), clamped at 6,
//             signed unless it rounds to 0.
//   stream    like the bf16 weight-streaming GEMM, with one lane taking the
//             16 code bytes of one block (32 k of one row; from LDS in the
//             main kernel, from global memory in the general one): the four
//             lanes of a row cover 128 consecutive k, and MFMA step u takes
//             code bytes 4u..4u+3 of every lane, converted with
//             v_cvt_scalef32_pk_bf16_fp4 (element 0 = low nibble, measured).
//             The token fragments are loaded at the same k, so both MFMA
//             operands agree on which 32 k a step sums over.
//
// A 16-byte code load carries 32 weights, so per code byte the token-fragment
// and scale loads weigh four times more than in the bf16 kernel, and a
// lane's codes in the MFMA layout cover only half of each 128-byte line.  The
// main kernel (stream_mx_lds_kernel) therefore copies the codes into LDS as
// whole lines with direct, non-temporal loads, copies the token tile into LDS
// once per work-group, and loads the scales of two 256-k stages with one
// 16-byte load per row.
#include <algorithm>

#include "gemm_problems.h"
#include "kernels.h"
#include "mxfp4_device.h"

namespace lmoe {

// E2M1 magnitude code of a = |w| / X in [0, 8): nearest of 0, 0.5, 1, 1.5, 2,
// 3, 4, 6, ties to the even code.  The thresholds are the midpoints between
// neighbours; at a midpoint the comparison is strict when the lower
// neighbour's code is even (0.25, 1.25, 2.5, 5) and not strict when the upper
// one's is (0.75, 1.75, 3.5).
__device__ __forceinline__ uint32_t e2m1_magnitude_code(float a) {
  return (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) +
         (a > 5.0f);
}

__global__ __launch_bounds__(256) void mxfp4_quantize_kernel(const uint16_t* __restrict__ w,
                                                             long nblocks,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  for (long b = (long)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks;
       b += (long)gridDim.x * blockDim.x) {
    float v[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(w + b * 32 + c * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[c * 8 + 2 * i] = __uint_as_float(q[i] << 16);
        v[c * 8 + 2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    int e = -127;
    if (amax > 0.f) {
      int ex;
      (void)frexpf(amax, &ex);  // amax = m 2^ex, 0.5 <= m < 1
      e = min(max(ex - 1 - 2, -127), 127);
    }
    u32x4 out;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = v[d * 8 + i];
        const uint32_t mag = e2m1_magnitude_code(ldexpf(fabsf(x), -e));
        const uint32_t code = mag | ((x < 0.f && mag) ? 8u : 0u);
        word |= code << (4 * i);
      }
      out[d] = word;
    }
    *reinterpret_cast<u32x4*>(codes + b * 16) = out;
    scales[b] = static_cast<uint8_t>(e + 127);
  }
}

hipError_t mxfp4_quantize(const uint16_t* w, long rows, int cols, uint8_t* codes,
                          uint8_t* scales, hipStream_t s) {
  const long nblocks = rows * (cols / 32);
  if (nblocks <= 0) return hipSuccess;
  const long grid = std::min<long>((nblocks + 255) / 256, 65536);
  mxfp4_quantize_kernel<<<grid, 256, 0, s>>>(w, nblocks, codes, scales);
  return hipGetLastError();
}

// General grouped expert GEMM over the 16-row tiles of the tile list (any K
// that is a multiple of 128).  Work-group = NW waves on RG*16 weight rows of
// one expert and one 16-row token tile; the k range is split over the waves
// (each a multiple of 128), partial sums added in LDS in a fixed order.  Per
// 128-k step a lane holds RG code blocks (16 bytes each), RG scale bytes and
// 4 token fragments; two steps in flight.
template <class P, int NW, int RG>
__global__ __launch_bounds__(NW * 64) void stream_mx_kernel(P p, const Tile* tiles,
                                                            const int* ntiles) {
  __shared__ f32x4 red[NW > 1 ? NW : 1][RG][64];
  const int nblocks = p.N() / (16 * RG);
  const int nb = blockIdx.x % nblocks;
  const int tm = blockIdx.x / nblocks;
  if (tm >= *ntiles) return;
  const Tile t = tiles[tm];
  const int e = t.expert, m0 = t.row0, mcount = t.nrows;
  const int n0 = nb * (16 * RG);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int kw = p.K() / NW;
  const int kbeg = w * kw;
  const int nit = kw / 128;

  const uint8_t* cw[RG];
  const uint8_t* sw[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    const int row = n0 + g * 16 + r16;
    cw[g] = p.codes_row(e, row) + kbeg / 2 + q * 16;
    sw[g] = p.scales_row(e, row) + kbeg / 32 + q;
  }
  // token rows past the tile's count read the tile's first row (not stored)
  const uint16_t* xr = p.a_row(m0 + (r16 < mcount ? r16 : 0)) + kbeg + q * 32;

  f32x4 acc[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 CA[RG], CB[RG];
  uint32_t SA[RG], SB[RG];
  bf16x8 XA[4], XB[4];
  auto load = [&](u32x4(&C)[RG], uint32_t(&S)[RG], bf16x8(&X)[4], int it) {
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      C[g] = *reinterpret_cast<const u32x4*>(cw[g] + it * 64);
      S[g] = sw[g][it * 4];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) X[u] = load8(xr + it * 128 + u * 8);
  };
  auto compute = [&](const u32x4(&C)[RG], const uint32_t(&S)[RG], const bf16x8(&X)[4]) {
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      const float sc = mx_scale(S[g]);
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[g] = mfma_bf16(mx_decode8(C[g][u], sc), X[u], acc[g]);
    }
  };
  if (nit > 0) load(CA, SA, XA, 0);
  for (int it = 0; it < nit; it += 2) {
    if (it + 1 < nit) load(CB, SB, XB, it + 1);
    compute(CA, SA, XA);
    if (it + 1 < nit) {
      if (it + 2 < nit) load(CA, SA, XA, it + 2);
      compute(CB, SB, XB);
    }
  }

  const int ncol = (lane >> 4) * 4;
  if constexpr (NW == 1) {
#pragma unroll
    for (int g = 0; g < RG; ++g)
      if (r16 < mcount) p.store(e, m0 + r16, n0 + g * 16 + ncol, acc[g]);
  } else {
#pragma unroll
    for (int g = 0; g < RG; ++g) red[w][g][lane] = acc[g];
    __syncthreads();
    for (int g = w; g < RG; g += NW) {
      f32x4 sm = red[0][g][lane];
#pragma unroll
      for (int v = 1; v < NW; ++v) sm += red[v][g][lane];
      if (r16 < mcount) p.store(e, m0 + r16, n0 + g * 16 + ncol, sm);
    }
  }
}

namespace {

typedef __attribute__((address_space(3))) void lds_dst_t;

// s_waitcnt with only the vector-memory counter set to N (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt and lgkmcnt left at their maximum).
template <int N>
__device__ __forceinline__ void vmem_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// raw buffer over 2 GiB from `base` (the hardware returns 0 past it)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFF0,
                                           0x00020000);
}

}  // namespace

// Grouped expert GEMM for K a multiple of 512 and N of 16 NW RG (codes and
// scales 16-byte aligned).  Work-group = NW waves on one 16-row token tile
// and 16 NW RG weight rows, each wave RG row groups (16 RG rows) over the
// whole k range, in stages of 256 k (launched with 4 waves of 2 or 4 row
// groups; 8 waves on 256 rows measured 1-2% slower: 332 vs 324 us for the
// decode batch's down projection).  Everything a stage needs from memory
// arrives by direct global -> LDS loads issued one stage ahead:
//  - each wave copies its own rows' codes of the stage (16 RG x 128 bytes,
//    2 RG loads of 8 whole lines) with the non-temporal hint into its own two
//    LDS slots.  Measured on the decode batch's up-projection codes with no
//    arithmetic: 7.1 TB/s, the read ceiling of the chip, against 6.2-6.3 TB/s
//    for these bytes loaded into registers 16 rows x 64 bytes at a time (the
//    MFMA layout, both halves of a line back to back) and 6.2-6.3 without the
//    hint;
//  - the stage's token tile (16 rows x 512 bytes) is copied by the whole
//    work-group, 8 / NW loads per wave;
//  - the scale bytes of a pair of stages come in one 16-byte register load per
//    row, one pair ahead.
// One barrier per stage.  LDS rows are XOR-swizzled: code row r keeps its
// 16-byte chunk c at c ^ (r % 8), token row t its chunk c at c ^ t.  Work
// items (tile, row block) are taken XCD-major.  The products and their order
// are those of the general kernel's k assignment: lane (r, q) of step u in
// half h of a stage takes code bytes 4u..4u+3 of block 4h + q of row r.
// LDS per work-group: 48 KB with 4 waves of 2 row groups (three work-groups
// per CU), 80 KB with 4 of 4 (two).
template <class P, int NW, int RG>
__device__ __forceinline__ void stream_mx_lds_body(const P& p, const Tile* tiles,
                                                   const int* ntiles) {
  constexpr int ROWS = NW * 16 * RG;
  static_assert(8 % NW == 0 && NW * 2 * 16 * RG * 128 + 2 * 16 * 512 <= 160 * 1024, "shape");
  constexpr int CSLOT = 16 * RG * 128;  // one wave's codes of one stage
  constexpr int TSLOT = 16 * 512;       // the token tile of one stage
  constexpr int TPW = 8 / NW;           // token loads (2 rows each) per wave
  __shared__ __attribute__((aligned(1024))) char smem[NW * 2 * CSLOT + 2 * TSLOT];

  const int nwg = p.N() / ROWS;
  const int nwork = __builtin_amdgcn_readfirstlane(*ntiles) * nwg;
  const int b = blockIdx.x;
  if (b >= nwork) return;
  const int per = nwork >> 3;
  const int item = b < (per << 3) ? (b & 7) * per + (b >> 3) : b;
  const int nb = item % nwg;
  const int tix = item / nwg;
  const int e = __builtin_amdgcn_readfirstlane(tiles[tix].expert);
  const int m0 = __builtin_amdgcn_readfirstlane(tiles[tix].row0);
  const int mcount = __builtin_amdgcn_readfirstlane(tiles[tix].nrows);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int nst = p.K() / 256;
  const int kb = p.K() / 2;  // code bytes per row
  const int n0 = nb * ROWS + w * 16 * RG;

  // code loads: load j fills this wave's rows 8j .. 8j + 7, lane l row
  // 8j + l / 8, LDS position l % 8 holding chunk (l % 8) ^ (row % 8)
  const char* cbase = reinterpret_cast<const char*>(p.codes_row(e, n0));
  const __amdgpu_buffer_rsrc_t rc = raw_buffer(cbase);
  const uint32_t coff = (uint32_t)((lane >> 3) * kb + (((lane & 7) ^ ((lane >> 3) & 7)) << 4));
  char* const cslots = smem + w * 2 * CSLOT;
  // token loads: load i of wave w fills token rows 2v and 2v + 1 (v = TPW w +
  // i), lane l row 2v + l / 32, LDS position l % 32 holding chunk (l % 32) ^
  // row; rows past the tile's count read its first row (never stored).
  // Offsets from the tile's first row are not negative: the dispatch keeps an
  // expert's rows in token order.
  const char* abase = reinterpret_cast<const char*>(p.a_row(m0));
  uint32_t toff[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int trow = 2 * (TPW * w + i) + (lane >> 5);
    const char* tsrc = reinterpret_cast<const char*>(p.a_row(m0 + (trow < mcount ? trow : 0)));
    toff[i] = (uint32_t)(tsrc - abase) + (uint32_t)(((lane & 31) ^ trow) << 4);
  }
  const __amdgpu_buffer_rsrc_t ra = raw_buffer(abase);
  char* const tslots = smem + NW * 2 * CSLOT;
  auto issue = [&](int st) __attribute__((always_inline)) {
    char* cs = cslots + (st & 1) * CSLOT;
#pragma unroll
    for (int j = 0; j < 2 * RG; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (lds_dst_t*)(cs + j * 1024), 16, coff,
                                               st * 128 + j * 8 * kb, 0, 2 /* nt */);
#pragma unroll
    for (int i = 0; i < TPW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (lds_dst_t*)(tslots + (st & 1) * TSLOT + (TPW * w + i) * 1024), 16, toff[i],
          st * 512, 0, 0);
  };
  const uint8_t* sw[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) sw[g] = p.scales_row(e, n0 + g * 16 + r16);
  u32x4 scur[RG], snext[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) snext[g] = *reinterpret_cast<const u32x4*>(sw[g]);
  f32x4 acc[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue(0);
  for (int st = 0; st < nst; ++st) {
    // this stage's loads (every wave's) have landed, and every wave is done
    // with the slots the next stage's loads overwrite
    vmem_wait<0>();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (st + 1 < nst) issue(st + 1);
    if ((st & 1) == 0) {
#pragma unroll
      for (int g = 0; g < RG; ++g) scur[g] = snext[g];
      if (st + 2 < nst) {
#pragma unroll
        for (int g = 0; g < RG; ++g)
          snext[g] = *reinterpret_cast<const u32x4*>(sw[g] + (st + 2) * 8);
      }
    }
    const char* cs = cslots + (st & 1) * CSLOT;
    const char* ts = tslots + (st & 1) * TSLOT;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        x[u] = *reinterpret_cast<const bf16x8*>(ts + r16 * 512 + (((h * 16 + q * 4 + u) ^ r16) << 4));
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        const int row = g * 16 + r16;
        const u32x4 c = *reinterpret_cast<const u32x4*>(cs + row * 128 + (((h * 4 + q) ^ (row & 7)) << 4));
        const float sc = mx_scale(__builtin_amdgcn_ubfe(scur[g][(st & 1) * 2 + h], q * 8, 8));
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[g] = mfma_bf16(mx_decode8(c[u], sc), x[u], acc[g]);
      }
    }
  }
  const int ncol = q * 4;
#pragma unroll
  for (int g = 0; g < RG; ++g)
    if (r16 < mcount) p.store(e, m0 + r16, n0 + g * 16 + ncol, acc[g]);
}

template <class P, int NW, int RG>
__global__ __launch_bounds__(NW * 64) void stream_mx_lds_kernel(P p, const Tile* tiles,
                                                                const int* ntiles) {
  stream_mx_lds_body<P, NW, RG>(p, tiles, ntiles);
}

// stream_mx_lds_kernel where its conditions hold (K a multiple of 512, N of
// 128, codes and scales 16-byte aligned, and the token rows' byte offsets
// from a tile's first row within the 2 GiB of a buffer descriptor, which
// holds while `a_rows` rows do: gathered rows (`a_rows` = the token count) are
// one expert's tokens in ascending order, so they lie after the first by less
// than the token count; rows read in place lie within the tile's 16);
// otherwise the general kernel with the largest of 4, 2, 1 waves per
// work-group whose k share is a whole number of 128-k steps (K is a multiple
// of 128).
// Four waves of two row groups (128 weight rows per work-group), or of four
// (256) when `wide` and N allows it: each work-group copies its tile's token
// rows once per stage, and with ~8 rows per expert those are a third of its
// bytes; measured standalone (us, T = 32 / T = 192): up projection 322-325 /
// 500-501 with two, 327-328 / 483-484 with four; down projection 328 / 473
// with two, 337 / 472 with four; eight waves of two or four were no better.
template <class P>
static hipError_t launch_mx(const P& p, const Tile* tiles, const int* ntiles, int max_tiles,
                            long a_rows, bool wide, hipStream_t s) {
  const bool aligned = ((reinterpret_cast<uintptr_t>(p.codes) | reinterpret_cast<uintptr_t>(p.scales)) & 15) == 0;
  const long a_span = a_rows * p.K() * 2;
  if (p.K() % 512 == 0 && p.N() % 128 == 0 && aligned && a_span < (1L << 31)) {
    if (wide && p.N() % 256 == 0) {
      const long grid = (long)max_tiles * (p.N() / 256);
      if (grid <= 0) return hipSuccess;
      stream_mx_lds_kernel<P, 4, 4><<<grid, 256, 0, s>>>(p, tiles, ntiles);
      return hipGetLastError();
    }
    const long grid = (long)max_tiles * (p.N() / 128);
    if (grid <= 0) return hipSuccess;
    stream_mx_lds_kernel<P, 4, 2><<<grid, 256, 0, s>>>(p, tiles, ntiles);
    return hipGetLastError();
  }
  constexpr int RG = 4;
  const long grid = (long)max_tiles * (p.N() / (16 * RG));
  if (grid <= 0) return hipSuccess;
  if (p.K() % (4 * 128) == 0)
    stream_mx_kernel<P, 4, RG><<<grid, 256, 0, s>>>(p, tiles, ntiles);
  else if (p.K() % (2 * 128) == 0)
    stream_mx_kernel<P, 2, RG><<<grid, 128, 0, s>>>(p, tiles, ntiles);
  else
    stream_mx_kernel<P, 1, RG><<<grid, 64, 0, s>>>(p, tiles, ntiles);
  return hipGetLastError();
}

hipError_t stream_mx_exp_up(const ExpUpMx& p, const Tile* tiles, const int* ntiles,
                            int max_tiles, int tokens, int rows_per_expert, hipStream_t s) {
  return launch_mx(p, tiles, ntiles, max_tiles, tokens, rows_per_expert > 2, s);
}
hipError_t stream_mx_exp_down(const ExpDownMx& p, const Tile* tiles, const int* ntiles,
                              int max_tiles, hipStream_t s) {
  return launch_mx(p, tiles, ntiles, max_tiles, 16, false, s);
}

}  // namespace lmoe
