// Internal launchers of libmoe.so. Each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ------------------------------------------------------------------ router
struct RouterArgs {
  const void *x;         // [T, d] act
  const float *w;        // [E, d]
  void *w_split;         // bf16 act: [3, E, d] bf16 planes of w (workspace)
  float *logits;         // [T, parts * E] partial logits (workspace)
  const float *bias;     // [E] or null
  int64_t T;
  int d, E, K;
  int mode;              // moe_route_mode
  int renormalize;
  float routed_scale;
  int32_t *idx;          // [T, K]
  float *g;              // [T, K]
  float *gap;            // [T] or null
  float *top;            // [T, K+1] or null
};
hipError_t launch_router(const RouterArgs &a, int act_bf16, hipStream_t s);
// True when the router runs one wavefront per token (few experts, a narrow
// model, little work; reads a.T, a.E, a.d) instead of the matrix-core GEMM.
bool router_valu(const RouterArgs &a);
// QuantileBalancer update (sigmoid routing): runs the router (a.top must be
// set: its column K is the threshold), then the differences diff [E, T],
// per-expert order statistics q [E] and the centred new_bias [E].
hipError_t launch_quantile_balance(const RouterArgs &a, int act_bf16, float *diff, float *q,
                                   float *new_bias, hipStream_t s);
// Router auxiliary losses (load-balancing loss and z-loss) of one step:
// runs the router, then per-chunk (16 to 64 tokens) partial sums into part
// [router_loss_chunks(T), E + 1] and the two losses into losses [2].
hipError_t launch_router_losses(const RouterArgs &a, int act_bf16, const int32_t *counts,
                                float alpha, float z_weight, float *part, float *losses,
                                hipStream_t s);
int64_t router_loss_chunks(int64_t T);
// Workspace of the router: split weight planes and partial logits.
inline size_t router_split_bytes(int64_t E, int64_t d, int act_bf16) {
  return act_bf16 ? static_cast<size_t>(3 * E * d * 2) : 0;
}
// K splits of the router GEMM: when the output tiles alone cannot fill the
// chip (few tokens, or few experts: E x 3 planes is a narrow output), the
// reduction over d is split and the partial logits are summed in fixed
// order by the selection kernel. At most 8 (the selection's bound) and d /
// 512. T <= 256: the generic kernel; bf16 planes with more tokens: the
// pipelined kernel's 128x128 tile, splits enough for ~384 workgroups (two
// per CU).
inline int router_splits(int64_t T, int64_t d, int64_t E, int act_bf16) {
  const int64_t smax = d / 512 < 1 ? 1 : (d / 512 > 8 ? 8 : d / 512);
  if (T <= 256) return static_cast<int>(smax);
  if (!act_bf16) return 1;
  const int64_t tiles = ((T + 127) / 128) * ((3 * E + 127) / 128);
  const int64_t s = (384 + tiles - 1) / tiles;
  return static_cast<int>(s < 1 ? 1 : (s > smax ? smax : s));
}
inline size_t router_logit_bytes(int64_t T, int64_t E, int64_t d, int act_bf16) {
  return static_cast<size_t>(T * E * (act_bf16 ? 3 : 1) * 4 *
                             router_splits(T, d, E, act_bf16));
}

// ------------------------------------------------------------------ dispatch
// Grouped-GEMM m-tile table entry: {expert, row_begin, row_end, group_first,
// group_size}; a group is a run of at most kTileGroup m-tiles of one expert.
constexpr int kTileInts = 5;
constexpr int kTileGroup = 8;
// Slots per histogram / scatter chunk.
constexpr int kChunkSlots = 1024;

__host__ __device__ inline int64_t n_chunks(int64_t slots) { return (slots + kChunkSlots - 1) / kChunkSlots; }

hipError_t launch_hist(const int32_t *idx, int64_t slots, int E, int32_t *chunk_hist,
                       hipStream_t s);

struct ScanArgs {
  const int32_t *chunk_hist;  // [n_chunks, E] in; becomes absolute bases
  int32_t *chunk_base;        // [n_chunks, E] out (may alias chunk_hist)
  int64_t slots;
  int E;
  int32_t *counts;            // [E]
  int32_t *offsets;           // [E+1]
  // grouped GEMM m-tile tables for tile heights bm / bm2 (tiles null -> skipped)
  int bm;
  int32_t *tiles;             // [max_tiles, kTileInts] (see below)
  int32_t *n_tiles;           // [1]
  int bm2;
  int32_t *tiles2;
  int32_t *n_tiles2;
  // near-tie count of the router gap (gap null -> skipped)
  const float *gap;
  int64_t T;
  float tie_eps;
  int32_t *n_near_ties;
};
hipError_t launch_scan(const ScanArgs &a, hipStream_t s);

// Tile table from existing offsets (for moe_expert_ffn).
hipError_t launch_tiles(const int32_t *offsets, int E, int bm, int32_t *tiles,
                        int32_t *n_tiles, hipStream_t s);

struct ScatterArgs {
  const int32_t *idx;
  const float *g;             // or null
  const int32_t *chunk_base;  // [n_chunks, E] absolute
  int64_t slots;
  int K, E;
  int32_t *perm, *sorted_token, *inv;
  float *sorted_w;            // or null
};
hipError_t launch_scatter(const ScatterArgs &a, hipStream_t s);

// Histogram, scan and scatter in one workgroup (same outputs as the three
// launches; chunk_hist / chunk_base unused) when dispatch_fused_ok().
constexpr int64_t kFusedMaxSlots = 16384;
bool dispatch_fused_ok(int64_t slots, int E);
hipError_t launch_dispatch_fused(const ScanArgs &a, const ScatterArgs &sc, hipStream_t s);

hipError_t launch_gather(const void *rows, const int32_t *sorted_token, int64_t n_rows,
                         int64_t row_bytes, void *out, hipStream_t s);

// ------------------------------------------------------------------ GEMM
// (EPI_GLU_F32, the persistent kernel only: the gate and up products of a
// SwiGLU tile stored in fp32, gate to out, up to out2)
enum Epilogue {
  EPI_SWIGLU = 0, EPI_SCALE = 1, EPI_STORE = 2, EPI_COMBINE = 3, EPI_STORE_F32 = 4,
  EPI_GLU_F32 = 5
};

// C = A B^T over one or two K segments, A [M, K] row-major (optionally row
// gathered), B [N, K] row-major ("out x in" weights), grouped by expert via a
// device tile table or dense.
struct GemmArgs {
  const void *a;
  int64_t lda;
  const int32_t *a_rows;     // gather: A row of tile row m is a_rows[m]
  const void *b0;            // B (gate for SWIGLU)
  const void *b1;            // up (SWIGLU only)
  int64_t ldb;
  int64_t b_stride;          // elements between experts' B matrices
  int K;
  const void *a2;            // second K segment (null: none)
  int64_t lda2;
  const void *b2;
  int64_t ldb2;
  int K2;
  int64_t M;                 // rows (dense)
  int N;                     // output columns
  const int32_t *tiles;      // grouped tile table, or null (dense)
  const int32_t *n_tiles;    // grouped: device count
  int64_t max_mtiles;        // bound on m tiles (grid size)
  void *out;
  int64_t ldo;
  const float *row_scale;    // SCALE (null -> 1)
  const void *y;             // COMBINE: routed rows [T*K, ldy]
  int64_t ldy;
  const int32_t *inv;
  int topk;
  int64_t a_extent;          // rows A may address (0: M; required for tile tables)
  int k_split;               // fp32-store only: K split count (0 or 1 = none);
  int64_t split_stride;      // elements between the splits' partial outputs
  int out_f32;               // SCALE: fp32 output instead of act dtype
  int64_t b2_stride;         // elements between experts' B matrices of the second K segment
  // K-grouped: tile table entries {expert, m_begin, m_end}
  // over the output rows; expert e reduces over columns [k_offsets[e],
  // k_offsets[e+1]) of A and B (multiples of 64, shared by all experts) and
  // writes its output at out + e * out_stride.
  const int32_t *k_offsets;
  int64_t out_stride;
  // B (and b2) stored K-major, [K, N] row-major with leading dimension ldb
  // (pipelined kernel, fp32-store epilogue, no gate/up pair)
  int b_kmajor;
  void *out2;                // GLU_F32: the up products (out: the gate products)
};

// Tile shapes (rows x B-rows per workgroup): SMALL_M 16x256, LARGE 128x128,
// WIDE 128x256, TALL 256x128, HUGE 256x256, MID 64x64, SMALL_N64 16x64,
// TALL_N64 128x64 (fp32 uses SMALL_M / LARGE only).
enum TileCfg {
  TILE_SMALL_M = 0, TILE_LARGE = 1, TILE_WIDE = 2, TILE_TALL = 3, TILE_HUGE = 4, TILE_MID = 5,
  TILE_SMALL_N64 = 6, TILE_TALL_N64 = 7
};
// Output tiles of a GEMM of `rows` x `n_out` under a tile shape (SwiGLU
// halves the B rows of a tile into output columns).
int64_t tile_count(int cfg, int64_t rows, int64_t n_out, int glu);
int tile_bm(int cfg);
int tile_bn(int cfg);
hipError_t launch_gemm(const GemmArgs &a, int epi, int cfg, int act_bf16, hipStream_t s);

// Pipelined bf16 GEMM (gemm2.hip): direct-to-LDS loads.
// (256x256: 8 wavefronts as 2 x 4 of 128x64 blocks; _TALLW: 4 x 2 of 64x128;
// 128x128 and 64x128 run 4 wavefronts (2 x 2) in at most 80 KB of LDS, so
// two workgroups can share a CU; _W8D4 / _W8D3: 8 wavefronts (4 x 2) with A
// 4 / 3 stages ahead; 32x256: 4 wavefronts (1 x 4) streaming the weights for
// few rows per expert.)
enum Tile2Cfg {
  TILE2_256x256 = 0, TILE2_256x256_TALLW = 4, TILE2_128x128 = 5, TILE2_64x128 = 6,
  TILE2_128x128_W8D4 = 9, TILE2_256x128_W8D3 = 10, TILE2_32x256_D2 = 14
};
bool gemm2_applicable(const GemmArgs &a, int epi);
int gemm2_bm(int cfg);
int gemm2_bn(int cfg);  // B rows per tile (output columns, or gate + up halves)
// b (optional, N > 0): a second problem of the same epilogue and tile
// shape, run in the same launch after a's tiles.
hipError_t launch_gemm2(const GemmArgs &a, int epi, int cfg, hipStream_t s,
                        const GemmArgs *b = nullptr);
// Whether launch_gemm2 runs the launch on the persistent 256x256 kernel (one
// workgroup per CU, each over a fixed list of tiles): one problem, a SwiGLU,
// row-scale, fp32-store or fp32 gate/up epilogue, a reduction of at least 5
// stages (K-grouped fp32 stores: any), at least two tiles per CU.
bool gemm2_persistent(const GemmArgs &a, int epi, int cfg, const GemmArgs *b = nullptr);
// Pipelined tile for rows x n_out over K (grouped over `groups` experts, or
// dense with groups = 0), with an optional dense rows2 x n_out2 problem in
// the same launch.
int gemm2_pick(int64_t rows, int64_t groups, int64_t K, int64_t n_out, int glu,
               int64_t rows2 = 0, int64_t n_out2 = 0);
// Dense GEMM with the kernel and tile shape chosen from the problem size.
hipError_t launch_dense(const GemmArgs &a, int epi, int act_bf16, hipStream_t s);

// ------------------------------------------------------------------ combine
// out[t] = sum_k y[inv[t*K+k]] (+ add[t], the shared experts' fp32 output,
// if given), at model width.
hipError_t launch_combine_sum(const void *y, const int32_t *inv, int64_t T, int K, int width,
                              void *out, int act_bf16, hipStream_t s,
                              const float *add = nullptr);
// r[t] = RMSNorm(sum_k y[inv[t*K+k]]) * gamma (latent), or the plain sum.
hipError_t launch_combine_latent(const void *y, const int32_t *inv, int64_t T, int K, int L,
                                 int has_rmsnorm, float eps, const float *gamma, void *r,
                                 int act_bf16, hipStream_t s);

// ------------------------------------------------------------------ backward
// Router gradient (router.hip): dr[p] for the sorted rows p of each token's
// selected experts from dg[p] (the routing weights' gradients), with a.idx,
// a.logits (of a router pass on the same x), bias, mode, scale as routed.
hipError_t launch_router_backward(const RouterArgs &a, int act_bf16, const int32_t *inv,
                                  const float *dg, float *dr, hipStream_t s);
// backward.hip
hipError_t launch_fill0(void *p, size_t bytes, hipStream_t s);
// dst[b * dst_bstride + c * dst_ld + col0 + r] = src[b][r][c] (act dtype) for
// batches b with active[b] != 0 (all if null)
hipError_t launch_transpose(const void *src, int64_t batches, int64_t R, int64_t C,
                            const int32_t *active, void *dst, int64_t dst_ld, int64_t dst_bstride,
                            int64_t col0, int act_bf16, hipStream_t s);
// rows (act dtype; gathered by row_index, scaled by row_scale, either optional) as
// columns of dst (ld ldd, a multiple of 8): column q = row q (dense, zeros
// from R up to Q, a bound of the columns written) or, grouped, the runs
// [poff[e], poff[e+1]) hold rows [off[e], off[e+1]) then zeros (Q bounds
// poff[G]); widths multiples of 8
hipError_t launch_cols(const void *src, int64_t ld_src, const int32_t *row_index,
                       const float *row_scale, int64_t R, int64_t C, const int32_t *off,
                       const int32_t *poff, int G, int64_t Q, void *dst, int64_t ldd,
                       int act_bf16, hipStream_t s);
// padded expert offsets and the K-grouped m-tile tables of heights M1, M2
hipError_t launch_kgroup(const int32_t *counts, int E, int M1, int M2, int bm, int32_t *poff,
                         int32_t *t1, int32_t *n1, int32_t *t2, int32_t *n2, hipStream_t s);
// h = SiLU(a) u and [da | du] (act dtype [R, 2f]) from a, u and W_down^T dy (fp32
// [R, f]) and the row weights gw (1 if null); dg[p] = <W_down^T dy, h> if dg;
// with D null, h only
hipError_t launch_bwd_rows(const float *A, const float *U, const float *D, const float *gw,
                           int64_t R, int f, void *H, void *dAU, float *dg, int act_bf16,
                           hipStream_t s);
// dx = sum_k dXs[inv] + dXsh + add2 + sum_k dr W_router rows (terms optional)
hipError_t launch_bwd_dx(const float *dXs, const float *dXsh, const float *add2,
                         const int32_t *inv, const int32_t *idx, const float *dr, const float *wr,
                         int64_t T, int K, int d, void *dx, int act_bf16, hipStream_t s);
// latent: R = sum_k Y[inv] (fp32), rinv, R' = R rinv gamma (bf16)
hipError_t launch_latent_fwd(const float *Y, const int32_t *inv, int64_t T, int K, int L,
                             int norm, float eps, const float *gamma, float *R, float *rinv,
                             void *Rp, int act_bf16, hipStream_t s);
// latent: RMSNorm backward dR (bf16) from dR' (fp32)
hipError_t launch_latent_bwd(const float *dRp, const float *R, const float *rinv,
                             const float *gamma, int64_t T, int L, int norm, void *dR,
                             int act_bf16, hipStream_t s);
// out[l] = sum_t A[t, l] B[t, l] sc[t] (part: [colsum_blocks(T), L] scratch)
int64_t colsum_blocks(int64_t T);
hipError_t launch_colsum(const float *A, const float *B, const float *sc, int64_t T, int L,
                         float *part, float *out, hipStream_t s);
// dW_router from the logit gradients dr per sorted row; rows of an expert are
// split over dwr_splits(E, d) blocks (part: dwr_part_bytes(E, d) scratch)
int dwr_splits(int E, int d);
size_t dwr_part_bytes(int E, int d);
hipError_t launch_bwd_dwr(const float *dr, const int32_t *stok, const int32_t *offsets,
                          const void *x, int E, int d, float *part, float *dwr, int act_bf16,
                          hipStream_t s);

// Bias-based balancer step (balance.hip); nk = tokens x top-k.
hipError_t launch_balance(int E, int64_t nk, const int32_t *counts, float alpha, float *bias,
                          hipStream_t s);

// Peak-rate microbenchmarks (peak.hip): mode 0/1 MFMA 16x16x32 / 32x32x16
// bf16, 2 LDS 16-byte reads, 3/4 MFMAs with 3 reads per 131072 flops, 5/6
// with 2; clk: int64 [2 groups] (shader cycles, 100 MHz ticks); sink:
// uint32 [groups x threads].
hipError_t launch_peak(int mode, int threads, int groups, int iters, int64_t *clk,
                       uint32_t *sink, hipStream_t s);

}  // namespace moe
