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
//   stream    like the bf16 weight-streaming GEMM, with one lane loading the
//             16 code bytes of one block (32 k of one row): the four lanes of
//             a row cover 128 consecutive k, and MFMA step u takes code bytes
//             4u..4u+3 of every lane, converted with
//             v_cvt_scalef32_pk_bf16_fp4 (element 0 = low nibble, measured).
//             The token fragments are loaded at the same k, so both MFMA
//             operands agree on which 32 k a step sums over.
//
// Streaming the codes at HBM speed is limited by the number of vector-memory
// instructions, not by bytes or arithmetic: a 16-byte code load carries 32
// weights, so per code byte the token-fragment and scale loads weigh four
// times more than in the bf16 kernel.  The main kernel therefore (a) loads
// both 64-byte halves of every 128-byte code line back to back (the two
// halves in separate steps let the line leave the cache in between, and the
// HBM traffic nearly doubles), (b) loads the scales of two 256-k stages with
// one 16-byte load per row, and (c) splits a work-group's waves over rows,
// not k, so the token tile is read once per work-group into LDS and shared.
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

// Grouped expert GEMM for K a multiple of 512 KS (codes and scales 16-byte
// aligned, N a multiple of (WPG / KS) RG 16).  Work-group = WPG waves on one
// 16-row token tile: WPG / KS row groups of RG * 16 weight rows, each split
// over KS waves along k (KS = 1: one wave per row group over the whole k
// range; KS > 1 shortens the work items, so that the last round of
// work-groups on the chip is short, and adds the k parts in LDS in a fixed
// order).  k runs in 256-k stages: per stage a lane loads RG x 2 code blocks
// (the two halves of each code line together) and reads its 4 x 2 token
// fragments from LDS; the stage's token tile (16 rows x 256 k for each k
// part) is copied into LDS by the whole work-group one stage ahead (double
// buffer, one barrier per stage), and the scales come one 16-byte load per
// row for a pair of stages, one pair ahead.  Work items (tile, row block) are
// taken XCD-major.
template <class P, int RG, int WPG, int KS>
__global__ __launch_bounds__(WPG * 64) void stream_mx_shared_kernel(P p, const Tile* tiles,
                                                                    const int* ntiles) {
  constexpr int XROW = 256 + 8;         // bf16 per LDS token row (16-byte pad: no bank conflicts)
  constexpr int XT = 16 * XROW;         // one k part's token tile
  constexpr int XP = KS * 512 / (WPG * 64);  // 16-byte token pieces per thread per stage
  constexpr int NRG = WPG / KS;         // row groups per work-group
  static_assert(XP >= 1 && XP * WPG * 64 == KS * 512 && NRG * KS == WPG, "WPG, KS");
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][KS * XT];

  // Consecutive blocks go to the 8 XCDs in turn; block b runs work item
  // (b % 8) * (n / 8) + b / 8 so that the items of one tile (consecutive)
  // share an XCD and its L2.  Only the live tiles' items are numbered.
  const int nwg = p.N() / (NRG * 16 * RG);
  const int nwork = *ntiles * nwg;
  const int b = blockIdx.x;
  if (b >= nwork) return;
  const int per = nwork >> 3;
  const int item = b < (per << 3) ? (b & 7) * per + (b >> 3) : b;
  const int nb = item % nwg;
  const Tile t = tiles[item / nwg];
  const int e = t.expert, m0 = t.row0, mcount = t.nrows;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int rgw = w / KS, kh = w % KS;  // this wave's row group and k part
  const int klen = p.K() / KS;
  const int nst = klen / 256;           // stages per k part (even)
  const int n0 = (nb * NRG + rgw) * (16 * RG);

  const uint8_t* cw[RG];
  const uint8_t* sw[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    const int row = n0 + g * 16 + r16;
    cw[g] = p.codes_row(e, row) + kh * (klen / 2) + q * 16;
    sw[g] = p.scales_row(e, row) + kh * (klen / 32);
  }
  // token rows past the tile's count copy the tile's first row (not stored)
  const uint16_t* xsrc[XP];
  int xdst[XP];
#pragma unroll
  for (int j = 0; j < XP; ++j) {
    const int gp = j * WPG * 64 + threadIdx.x;
    const int part = gp / 512, piece = gp % 512;
    const int row = piece >> 5, col = (piece & 31) * 8;
    xsrc[j] = p.a_row(m0 + (row < mcount ? row : 0)) + part * klen + col;
    xdst[j] = part * XT + row * XROW + col;
  }
  const int xrd = kh * XT + r16 * XROW + q * 32;

  f32x4 acc[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 CA[2][RG], CB[2][RG];  // code blocks of two stages, [half][row group]
  u32x4 S0[RG], S1[RG];        // scale bytes of the current and the next stage pair
  bf16x8 XG[XP];               // token pieces on their way to LDS
  auto load_codes = [&](u32x4(&C)[2][RG], int st) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int g = 0; g < RG; ++g)
        C[h][g] = *reinterpret_cast<const u32x4*>(cw[g] + st * 128 + h * 64);
  };
  auto load_scales = [&](u32x4(&S)[RG], int st) {
#pragma unroll
    for (int g = 0; g < RG; ++g) S[g] = *reinterpret_cast<const u32x4*>(sw[g] + st * 8);
  };
  auto load_tokens = [&](int st) {
#pragma unroll
    for (int j = 0; j < XP; ++j) XG[j] = load8(xsrc[j] + st * 256);
  };
  auto store_tokens = [&](int buf) {
#pragma unroll
    for (int j = 0; j < XP; ++j) *reinterpret_cast<bf16x8*>(&xs[buf][xdst[j]]) = XG[j];
  };
  // one stage: scale byte q of dword 2*odd + h is the scale of this lane's
  // block in half h of the stage
  auto compute = [&](const u32x4(&C)[2][RG], int buf, int odd) {
    bf16x8 X[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        X[h][u] = *reinterpret_cast<const bf16x8*>(&xs[buf][xrd + h * 128 + u * 8]);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        const float sc = mx_scale(__builtin_amdgcn_ubfe(S0[g][odd * 2 + h], q * 8, 8));
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[g] = mfma_bf16(mx_decode8(C[h][g][u], sc), X[h][u], acc[g]);
      }
  };

  load_tokens(0);
  load_codes(CA, 0);
  load_scales(S0, 0);
  store_tokens(0);
  load_tokens(1);
  __syncthreads();
  for (int st = 0; st < nst; st += 2) {
    const bool more = st + 2 < nst;
    load_codes(CB, st + 1);
    if (more) load_scales(S1, st + 2);
    compute(CA, 0, 0);
    store_tokens(1);
    if (more) load_tokens(st + 2);
    __syncthreads();
    if (more) load_codes(CA, st + 2);
    compute(CB, 1, 1);
    if (more) {
      store_tokens(0);
      load_tokens(st + 3);
#pragma unroll
      for (int g = 0; g < RG; ++g) S0[g] = S1[g];
    }
    __syncthreads();
  }

  const int ncol = q * 4;
  if constexpr (KS == 1) {
#pragma unroll
    for (int g = 0; g < RG; ++g)
      if (r16 < mcount) p.store(e, m0 + r16, n0 + g * 16 + ncol, acc[g]);
  } else {
    // k parts added in part order (deterministic)
    __shared__ f32x4 red[KS][NRG][RG][64];
#pragma unroll
    for (int g = 0; g < RG; ++g) red[kh][rgw][g][lane] = acc[g];
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        f32x4 sm = red[0][rgw][g][lane];
#pragma unroll
        for (int v = 1; v < KS; ++v) sm += red[v][rgw][g][lane];
        if (r16 < mcount) p.store(e, m0 + r16, n0 + g * 16 + ncol, sm);
      }
    }
  }
}

// The shared-token kernel where its conditions hold; otherwise the general
// kernel with the largest of 4, 2, 1 waves per work-group whose k share is a
// whole number of 128-k steps (K is a multiple of 128).
template <class P>
static hipError_t launch_mx(const P& p, const Tile* tiles, const int* ntiles, int max_tiles,
                            hipStream_t s) {
  constexpr int kSharedRG = 2, kSharedWPG = 8;
  const bool aligned = ((reinterpret_cast<uintptr_t>(p.codes) | reinterpret_cast<uintptr_t>(p.scales)) & 15) == 0;
  if (p.K() % 512 == 0 && p.N() % (kSharedWPG * 16 * kSharedRG) == 0 && aligned) {
    // long k ranges (the down projection, k = 5120) in two parts: measured at
    // the decode batch 0.403 vs 0.435 ms (the work-groups' last round on the
    // chip is shorter); the up projection (k = 2048) is not faster that way
    if (p.K() >= 4096 && p.K() % 1024 == 0) {
      const long grid = (long)max_tiles * (p.N() / (kSharedWPG / 2 * 16 * kSharedRG));
      if (grid <= 0) return hipSuccess;
      stream_mx_shared_kernel<P, kSharedRG, kSharedWPG, 2><<<grid, kSharedWPG * 64, 0, s>>>(p, tiles, ntiles);
      return hipGetLastError();
    }
    const long grid = (long)max_tiles * (p.N() / (kSharedWPG * 16 * kSharedRG));
    if (grid <= 0) return hipSuccess;
    stream_mx_shared_kernel<P, kSharedRG, kSharedWPG, 1><<<grid, kSharedWPG * 64, 0, s>>>(p, tiles, ntiles);
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
                            int max_tiles, hipStream_t s) {
  return launch_mx(p, tiles, ntiles, max_tiles, s);
}
hipError_t stream_mx_exp_down(const ExpDownMx& p, const Tile* tiles, const int* ntiles,
                              int max_tiles, hipStream_t s) {
  return launch_mx(p, tiles, ntiles, max_tiles, s);
}

}  // namespace lmoe
