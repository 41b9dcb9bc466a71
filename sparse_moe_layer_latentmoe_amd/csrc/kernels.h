// Host-side launchers of the gfx950 kernels (each defined next to its kernel).
// All launchers enqueue on `s` and return hipGetLastError() of the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmoe {

struct ProjIn;
struct ProjOut;
struct ExpUp;
struct ExpDown;
struct ExpUpMx;
struct ExpDownMx;
struct Tile;

// Weight-streaming GEMMs (few tokens; expert tiles of 16 rows).
hipError_t stream_proj_in(const ProjIn& p, hipStream_t s);
hipError_t stream_proj_out(const ProjOut& p, hipStream_t s);
hipError_t stream_exp_up(const ExpUp& p, const Tile* tiles, const int* ntiles, int max_tiles,
                         hipStream_t s);
// rows_per_expert: the batch's average rows per expert, ceil(T K / E) (it
// picks the launch shape)
hipError_t stream_exp_down(const ExpDown& p, const Tile* tiles, const int* ntiles, int max_tiles,
                           int rows_per_expert, hipStream_t s);
constexpr int kStreamTileM = 16;
// Dense GEMMs stream weights for batches of at most this many tokens.
constexpr int kStreamDenseMaxTokens = 64;

// LDS-tiled MFMA GEMMs (many tokens; expert tiles of tiled_block_m() rows;
// every N must be a multiple of tiled_block_n()).
hipError_t tiled_proj_in(const ProjIn& p, hipStream_t s);
hipError_t tiled_proj_out(const ProjOut& p, hipStream_t s);
// tokens: the batch's token count (every gathered latent row index is below it)
hipError_t tiled_exp_up(const ExpUp& p, const Tile* tiles, const int* ntiles, int max_tiles,
                        int tokens, hipStream_t s);
hipError_t tiled_exp_down(const ExpDown& p, const Tile* tiles, const int* ntiles, int max_tiles,
                          hipStream_t s);
int tiled_block_m();
int tiled_block_n();

// Split-k LDS-tiled dense GEMMs for mid-sized batches (T <= kSplitMaxTokens):
// up to kSplitMax fp32 partial [T, N] arrays in `part`, then a fixed-order
// reduction that runs the problem's epilogue.  Same dimension requirements as
// the tiled GEMMs.
constexpr int kSplitMax = 8;
constexpr int kSplitMaxTokens = 256;
hipError_t split_proj_in(const ProjIn& p, float* part, hipStream_t s);
hipError_t split_proj_out(const ProjOut& p, float* part, hipStream_t s);

// MXFP4 expert weights: quantiser (rows x cols bf16 -> codes rows x cols/2,
// scales rows x cols/32; cols a multiple of 32) and the weight-streaming
// expert GEMMs (K a multiple of 128, N a multiple of 64).
hipError_t mxfp4_quantize(const uint16_t* w, long rows, int cols, uint8_t* codes,
                          uint8_t* scales, hipStream_t s);
// tokens as for tiled_exp_up, rows_per_expert as for stream_exp_down
hipError_t stream_mx_exp_up(const ExpUpMx& p, const Tile* tiles, const int* ntiles,
                            int max_tiles, int tokens, int rows_per_expert, hipStream_t s);
hipError_t stream_mx_exp_down(const ExpDownMx& p, const Tile* tiles, const int* ntiles,
                              int max_tiles, hipStream_t s);
// The LDS-tiled expert GEMMs with MXFP4 weights (large batches; same
// dimension requirements and tile list as tiled_exp_up / tiled_exp_down).
hipError_t tiled_mx_exp_up(const ExpUpMx& p, const Tile* tiles, const int* ntiles, int max_tiles,
                           int tokens, hipStream_t s);
hipError_t tiled_mx_exp_down(const ExpDownMx& p, const Tile* tiles, const int* ntiles,
                             int max_tiles, hipStream_t s);

// Router: fp32 logits, then per token sigmoid / bias / top-K / weights.  The
// logits GEMM may split k over router_splits(T, E, R) partial [T, E] arrays
// (logits must hold that many); router_select adds them in split order.
// Splitting happens only for T <= router_split_max_tokens(), into at most
// router_max_splits() parts.
constexpr int router_max_splits() { return 8; }
constexpr int router_split_max_tokens() { return 1024; }
int router_splits(int T, int E, int R);
hipError_t router_logits(const float* z, const float* wg, float* logits, int T, int E, int R,
                         hipStream_t s);
// n_group > 1: group-limited selection (at most 64 groups, one per lane).
hipError_t router_select(const float* logits, const float* bias, int T, int E, int R, int K,
                         int n_group, int topk_group, float rho, int32_t* idx, float* w,
                         hipStream_t s);

// Grouping by expert: counts[E], offsets[E+1], rows_tok[T*K], inv[T*K] and
// the tile list (tiles of at most tile_m rows) with its length in *ntiles.
// blockcnt is scratch of ceil(T/64) * E ints.
hipError_t dispatch(const int32_t* idx, int T, int K, int E, int32_t* blockcnt, int32_t* counts,
                    int32_t* offsets, int32_t* rows_tok, int32_t* inv, Tile* tiles,
                    int32_t* ntiles, int tile_m, hipStream_t s);

// The block's pre-norm for T tokens of width D (a multiple of 8): xt =
// bf16(gamma * h) [T, D] and rn = 1 / sqrt(mean(h^2) + eps) [T].
hipError_t prenorm(const uint16_t* h, const uint16_t* gamma, int T, int D, float eps,
                   uint16_t* xt, float* rn, hipStream_t s);

// r = sum_k w[t][k] O[inv[t][k]] -> r16 (bf16) and, if r32 != NULL, fp32.
hipError_t combine(const uint16_t* o, const int32_t* inv, const float* w, int T, int K, int R,
                   uint16_t* r16, float* r32, hipStream_t s);

}  // namespace lmoe
