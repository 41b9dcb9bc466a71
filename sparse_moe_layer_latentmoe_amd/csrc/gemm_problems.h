// The four bf16 GEMMs of the LatentMoE layer, described for the two GEMM
// kernels (weight streaming and LDS-tiled).  Every GEMM computes
//     C[m][n] = sum_k A[m][k] * B[n][k]
// with A the activations (row m) and B a weight stored out x in (row n), both
// contiguous along k, and fp32 accumulation.  A problem says where row m of A
// and row n of B start, for up to two consecutive k segments (k < K0 and
// k >= K0), the segment bases and row strides of A when its rows are strided
// (a_base*/lda*; a_row*(m) == a_base*() + m * lda*()), and otherwise gathered
// (kGatherA), the row strides of B (ldb*), and what the epilogue stores for
// four consecutive columns.
#pragma once
#include "lmoe_device.h"

namespace lmoe {

// [z | Hs] = x [W1 ; Wsu]^T  (fc1_latent and the shared expert's up
// projection share the input x; page "Nemotron 3 Ultra 架构深度拆解报告",
// CH5 §5.6 Steps 5 and 7).  Global column n < R gives the latent z, stored
// fp32 (router input) and bf16 (expert input); n >= R gives the shared
// expert's hidden relu(.)^2 in bf16.  One launch covers the columns
// [noff, noff + ncount), so the latent and the shared part can run as two
// launches on two streams (R is a multiple of every column block).  With the
// block's pre-norm fused, x holds bf16(gamma * h) and rscale[m] (the token's
// 1 / rms) multiplies row m's fp32 sums before the epilogue.
struct ProjIn {
  const uint16_t* x;
  const uint16_t* w1;
  const uint16_t* wsu;
  float* z32;
  uint16_t* z16;
  uint16_t* hs;
  int T, D, R, S;
  int noff, ncount;
  const float* rscale;  // [T] or null
  static constexpr bool kGatherA = false;
  static constexpr bool kStagedStore = false;
  __device__ const uint16_t* a_base0() const { return x; }
  __device__ const uint16_t* a_base1() const { return x; }
  __device__ long lda0() const { return D; }
  __device__ long lda1() const { return D; }
  __device__ long ldb0() const { return D; }
  __device__ long ldb1() const { return D; }
  __host__ __device__ int N() const { return ncount; }
  __host__ __device__ int K() const { return D; }
  __host__ __device__ int K0() const { return D; }
  __device__ const uint16_t* b_row0(int, int n) const {
    const int g = noff + n;
    return g < R ? w1 + (size_t)g * D : wsu + (size_t)(g - R) * D;
  }
  __device__ const uint16_t* b_row1(int, int) const { return nullptr; }
  __device__ const uint16_t* a_row0(int m) const { return x + (size_t)m * D; }
  __device__ const uint16_t* a_row1(int) const { return nullptr; }
  __device__ void store(int, int m, int n, f32x4 v) const {
    const int g = noff + n;
    if (rscale) v *= rscale[m];
    if (g < R) {
      *reinterpret_cast<f32x4*>(z32 + (size_t)m * R + g) = v;
      store4_bf16(z16 + (size_t)m * R + g, v);
    } else {
      store4_bf16_relu_sq(hs + (size_t)m * S + (g - R), v);
    }
  }
};

// y = [r | Hs] [W2 | Wsd]^T  (fc2_latent plus the shared expert's down
// projection, Step 7: the routed and shared outputs are added, so one GEMM
// over the concatenated k range gives their sum with a single rounding).
// With the block's residual fused, resid (the block input h, bf16 [T, D]) is
// added to the fp32 sums before that rounding.
// The same sum in two launches (part 1 then part 2, weight-streaming path):
// part 1 computes only Hs Wsd^T into ys (fp32 [T, D]); part 2 only r W2^T,
// adds ys (and resid) to its fp32 sums and rounds once.  part 0: both at once.
struct ProjOut {
  const uint16_t* r16;
  const uint16_t* hs;
  const uint16_t* w2;
  const uint16_t* wsd;
  uint16_t* y;
  int T, D, R, S;
  const uint16_t* resid;  // [T, D] or null
  int part = 0;
  float* ys = nullptr;    // [T, D] fp32 for parts 1 and 2
  static constexpr bool kGatherA = false;
  static constexpr bool kStagedStore = false;
  __device__ const uint16_t* a_base0() const { return part == 1 ? hs : r16; }
  __device__ const uint16_t* a_base1() const { return hs; }
  __device__ long lda0() const { return part == 1 ? S : R; }
  __device__ long lda1() const { return S; }
  __device__ long ldb0() const { return part == 1 ? S : R; }
  __device__ long ldb1() const { return S; }
  __host__ __device__ int N() const { return D; }
  __host__ __device__ int K() const { return part == 0 ? R + S : (part == 1 ? S : R); }
  __host__ __device__ int K0() const { return part == 0 ? R : K(); }
  __device__ const uint16_t* b_row0(int, int n) const {
    return part == 1 ? wsd + (size_t)n * S : w2 + (size_t)n * R;
  }
  __device__ const uint16_t* b_row1(int, int n) const { return wsd + (size_t)n * S; }
  __device__ const uint16_t* a_row0(int m) const {
    return part == 1 ? hs + (size_t)m * S : r16 + (size_t)m * R;
  }
  __device__ const uint16_t* a_row1(int m) const { return hs + (size_t)m * S; }
  __device__ void store(int, int m, int n, f32x4 v) const {
    if (part == 1) {
      *reinterpret_cast<f32x4*>(ys + (size_t)m * D + n) = v;
      return;
    }
    if (part == 2) v += *reinterpret_cast<const f32x4*>(ys + (size_t)m * D + n);
    if (resid) {
      const u16x4 h = *reinterpret_cast<const u16x4*>(resid + (size_t)m * D + n);
      v[0] += bf16_to_f32(h[0]);
      v[1] += bf16_to_f32(h[1]);
      v[2] += bf16_to_f32(h[2]);
      v[3] += bf16_to_f32(h[3]);
    }
    store4_bf16(y + (size_t)m * D + n, v);
  }
};

// Expert up projection + relu^2 (Step 6), grouped by expert: row p of the
// expert-sorted slot list reads the bf16 latent of token rows_tok[p].
struct ExpUp {
  const uint16_t* z16;
  const int32_t* rows_tok;
  const uint16_t* wup;  // [E, F, R]
  uint16_t* h;          // [slots, F]
  int R, F;
  static constexpr bool kGatherA = true;
  __device__ const uint16_t* a_base0() const { return z16; }
  __device__ const uint16_t* a_base1() const { return z16; }
  __device__ long lda0() const { return R; }
  __device__ long lda1() const { return R; }
  __device__ long ldb0() const { return R; }
  __device__ long ldb1() const { return R; }
  __host__ __device__ int N() const { return F; }
  __host__ __device__ int K() const { return R; }
  __host__ __device__ int K0() const { return R; }
  __device__ const uint16_t* b_row0(int e, int n) const {
    return wup + ((size_t)e * F + n) * R;
  }
  __device__ const uint16_t* b_row1(int, int) const { return nullptr; }
  __device__ const uint16_t* a_row0(int p) const { return z16 + (size_t)rows_tok[p] * R; }
  __device__ const uint16_t* a_row1(int) const { return nullptr; }
  __device__ void store(int, int p, int n, f32x4 v) const {
    store4_bf16_relu_sq(h + (size_t)p * F + n, v);
  }
  // non-temporal: for the weight-streaming kernel (few rows per expert)
  __device__ void store_nt(int, int p, int n, f32x4 v) const {
    store4_bf16_relu_sq_nt(h + (size_t)p * F + n, v);
  }
  // the same values in two steps, for output staged through LDS: pack4
  // gives the stored bits of four columns, store8 writes eight columns
  static constexpr bool kStagedStore = true;
  __device__ u16x4 pack4(f32x4 v) const { return pack4_bf16_relu_sq(v); }
  __device__ void store8(int p, int n, u16x8 v) const {
    *reinterpret_cast<u16x8*>(h + (size_t)p * F + n) = v;
  }
  __device__ void store8_nt(int p, int n, u16x8 v) const {
    __builtin_nontemporal_store(v, reinterpret_cast<u16x8*>(h + (size_t)p * F + n));
  }
};

// Expert down projection (Step 6): O[p] = H[p] Wdn[e]^T, stored bf16; the
// routing weight is applied by the combine.
struct ExpDown {
  const uint16_t* h;    // [slots, F]
  const uint16_t* wdn;  // [E, R, F]
  uint16_t* o;          // [slots, R]
  int R, F;
  static constexpr bool kGatherA = false;
  __device__ const uint16_t* a_base0() const { return h; }
  __device__ const uint16_t* a_base1() const { return h; }
  __device__ long lda0() const { return F; }
  __device__ long lda1() const { return F; }
  __device__ long ldb0() const { return F; }
  __device__ long ldb1() const { return F; }
  __host__ __device__ int N() const { return R; }
  __host__ __device__ int K() const { return F; }
  __host__ __device__ int K0() const { return F; }
  __device__ const uint16_t* b_row0(int e, int n) const {
    return wdn + ((size_t)e * R + n) * F;
  }
  __device__ const uint16_t* b_row1(int, int) const { return nullptr; }
  __device__ const uint16_t* a_row0(int p) const { return h + (size_t)p * F; }
  __device__ const uint16_t* a_row1(int) const { return nullptr; }
  __device__ void store(int, int p, int n, f32x4 v) const {
    store4_bf16(o + (size_t)p * R + n, v);
  }
  __device__ void store_nt(int, int p, int n, f32x4 v) const {
    store4_bf16_nt(o + (size_t)p * R + n, v);
  }
  static constexpr bool kStagedStore = true;
  __device__ u16x4 pack4(f32x4 v) const { return pack4_bf16(v); }
  __device__ void store8(int p, int n, u16x8 v) const {
    *reinterpret_cast<u16x8*>(o + (size_t)p * R + n) = v;
  }
  __device__ void store8_nt(int p, int n, u16x8 v) const {
    __builtin_nontemporal_store(v, reinterpret_cast<u16x8*>(o + (size_t)p * R + n));
  }
};

// Expert GEMMs with MXFP4 weights (block-scaled FP4; the layout of
// lmoe_quantize_mxfp4): weight row n of expert e is K/2 code bytes (element
// 2i in the low nibble of byte i) and K/32 scale bytes (2^(byte - 127) per
// block of 32 consecutive k).  Activations stay bf16.
struct ExpUpMx {
  const uint16_t* z16;
  const int32_t* rows_tok;
  const uint8_t* codes;   // [E, F, R/2]
  const uint8_t* scales;  // [E, F, R/32]
  uint16_t* h;            // [slots, F]
  int R, F;
  static constexpr bool kGatherA = true;
  __host__ __device__ int N() const { return F; }
  __host__ __device__ int K() const { return R; }
  __device__ const uint8_t* codes_row(int e, int n) const {
    return codes + ((size_t)e * F + n) * (R / 2);
  }
  __device__ const uint8_t* scales_row(int e, int n) const {
    return scales + ((size_t)e * F + n) * (R / 32);
  }
  __device__ const uint16_t* a_row(int p) const { return z16 + (size_t)rows_tok[p] * R; }
  __device__ void store(int, int p, int n, f32x4 v) const {
    store4_bf16_relu_sq(h + (size_t)p * F + n, v);
  }
  static constexpr bool kStagedStore = true;
  __device__ u16x4 pack4(f32x4 v) const { return pack4_bf16_relu_sq(v); }
  __device__ void store8(int p, int n, u16x8 v) const {
    *reinterpret_cast<u16x8*>(h + (size_t)p * F + n) = v;
  }
};

struct ExpDownMx {
  const uint16_t* h;      // [slots, F]
  const uint8_t* codes;   // [E, R, F/2]
  const uint8_t* scales;  // [E, R, F/32]
  uint16_t* o;            // [slots, R]
  int R, F;
  static constexpr bool kGatherA = false;
  __host__ __device__ int N() const { return R; }
  __host__ __device__ int K() const { return F; }
  __device__ const uint8_t* codes_row(int e, int n) const {
    return codes + ((size_t)e * R + n) * (F / 2);
  }
  __device__ const uint8_t* scales_row(int e, int n) const {
    return scales + ((size_t)e * R + n) * (F / 32);
  }
  __device__ const uint16_t* a_row(int p) const { return h + (size_t)p * F; }
  __device__ void store(int, int p, int n, f32x4 v) const {
    store4_bf16(o + (size_t)p * R + n, v);
  }
  static constexpr bool kStagedStore = true;
  __device__ u16x4 pack4(f32x4 v) const { return pack4_bf16(v); }
  __device__ void store8(int p, int n, u16x8 v) const {
    *reinterpret_cast<u16x8*>(o + (size_t)p * R + n) = v;
  }
};

// Split-k view of a dense problem for the LDS-tiled kernel: work-group
// (x, y) computes tile x of P over the k range [y * klen, (y + 1) * klen) and
// its epilogue writes fp32 partial sums to part[y][m][n] (mrows rows).  The
// split index is blockIdx.y, so the tiled kernel runs unchanged on a 2-D
// grid.  Both k segments of P are handled: K0 of the view is where P's
// segment boundary falls inside the range (clamped to [0, klen]), and each
// segment's pointers are advanced to the range start.  klen and P's K0 are
// multiples of the k tile, so no k tile straddles the boundary.
template <class P>
struct SplitK {
  P p;
  int klen;
  float* part;
  int mrows;
  static constexpr bool kGatherA = P::kGatherA;
  static constexpr bool kStagedStore = false;
  __device__ int kstart() const { return blockIdx.y * klen; }
  __device__ int off1() const {
    const int v = kstart() - p.K0();
    return v < 0 ? 0 : v;
  }
  __device__ const uint16_t* a_base0() const { return p.a_base0() + kstart(); }
  __device__ const uint16_t* a_base1() const { return p.a_base1() + off1(); }
  __device__ long lda0() const { return p.lda0(); }
  __device__ long lda1() const { return p.lda1(); }
  __device__ long ldb0() const { return p.ldb0(); }
  __device__ long ldb1() const { return p.ldb1(); }
  __host__ __device__ int N() const { return p.N(); }
  __host__ __device__ int K() const { return klen; }
  __device__ int K0() const {
    const int v = p.K0() - kstart();
    return v < 0 ? 0 : (v > klen ? klen : v);
  }
  __device__ const uint16_t* b_row0(int e, int n) const { return p.b_row0(e, n) + kstart(); }
  __device__ const uint16_t* b_row1(int e, int n) const {
    const uint16_t* q = p.b_row1(e, n);
    return q ? q + off1() : nullptr;
  }
  __device__ const uint16_t* a_row0(int m) const { return p.a_row0(m) + kstart(); }
  __device__ const uint16_t* a_row1(int m) const {
    const uint16_t* q = p.a_row1(m);
    return q ? q + off1() : nullptr;
  }
  __device__ void store(int, int m, int n, f32x4 v) const {
    *reinterpret_cast<f32x4*>(part + ((size_t)blockIdx.y * mrows + m) * p.N() + n) = v;
  }
};

}  // namespace lmoe
