// Backward pass of the layer (bf16 or fp32 activations): the elementwise,
// transpose and reduction kernels around the GEMMs that api.hip enqueues.
//
// The layer (APEX-1 Mathematical Reference - Part 3, 13.2 and 12.2) is
// y_t = sum_s FFN_s(x_t) + sum_k g_k FFN_{e_k}(x_t), FFN(x) = W_down h,
// h = SiLU(a) * u, a = W_gate x, u = W_up x. For an output gradient dy:
//   dh = g W_down^T dy,   dg_k = <dy, FFN_{e_k}(x)> = <W_down^T dy, h>,
//   da = dh * u * SiLU'(a),  du = dh * SiLU(a),  SiLU' = s (1 + a (1 - s)),
//   dx += W_gate^T da + W_up^T du,
//   dW_down += (g dy) h^T,  dW_gate += da x^T,  dW_up += du x^T,
// and the router gradient from dg (router.hip). The selection passes no
// gradient and the balance bias gets none; experts no token selected get no
// weight gradient ("StableLatentMoE and QuantileBalancer": inactive experts'
// gradients stay unset).
//
// Every product runs as an NT GEMM (C = A B^T, both operands K-contiguous;
// bf16: the pipelined kernel, fp32: the generic one). Products whose natural
// operand is K-strided use transposed copies: the weights of active experts
// (W_down^T, W_gate^T, W_up^T) and, for
// the weight gradients, the activations in expert-contiguous columns whose
// per-expert runs are padded to multiples of 64 with zeros (the K-grouped
// GEMM reduces each expert over its own run).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void fill0_kernel(uint4 *p, int64_t n16) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n16;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// 64 x 64 element tiles (bf16 or fp32 bits: E = uint16_t or uint32_t) through
// LDS with 16-byte global accesses on both sides: tile row i holds 64
// consecutive columns of one source row; a destination row takes EPC tile
// rows of one column per 16-byte chunk. Widths and offsets are multiples of
// 8 elements. The 16-byte chunks of row r sit XOR-swizzled by (r / EPC) so
// that a wavefront's column reads (EPC-row groups x a few columns) fall in
// distinct LDS banks, as its row writes do.
template <typename E>
struct TileOf {
  static constexpr int EPC = 16 / static_cast<int>(sizeof(E));  // elements per chunk
  static constexpr int CPR = 64 / EPC;                           // chunks per tile row
  static constexpr int P = 64;                                   // pitch (elements)
  // element offset in row r of logical column c
  static __device__ __forceinline__ int col(int r, int c) {
    return (((c / EPC) ^ ((r / EPC) & (CPR - 1))) * EPC) + c % EPC;
  }
};
template <typename E> struct ChunkT;
template <> struct ChunkT<uint16_t> { using C = Chunk<bf16_t>; };
template <> struct ChunkT<uint32_t> { using C = Chunk<float>; };

template <typename E>
__device__ __forceinline__ void tile_store_cols(const E (*tile)[TileOf<E>::P], int64_t c0,
                                                int64_t C, int64_t q0, int64_t Q, E *dst,
                                                int64_t dst_ld) {
  constexpr int EPC = TileOf<E>::EPC, CPR = TileOf<E>::CPR;
  for (int i = threadIdx.x; i < 64 * CPR; i += 256) {
    const int c = i / CPR, qc = i % CPR;
    if (c0 + c >= C || q0 + EPC * qc >= Q) continue;
    union {
      uint4 v;
      E e[EPC];
    } u;
#pragma unroll
    for (int j = 0; j < EPC; ++j) u.e[j] = tile[EPC * qc + j][TileOf<E>::col(EPC * qc + j, c)];
    *reinterpret_cast<uint4 *>(dst + (c0 + c) * dst_ld + q0 + EPC * qc) = u.v;
  }
}

// dst[b * dst_bstride + c * dst_ld + col0 + r] = src[b][r][c]; batches b with
// active && !active[b] are skipped.
template <typename E>
__global__ __launch_bounds__(256) void transpose_kernel(const E *src, int64_t R, int64_t C,
                                                        const int32_t *active, E *dst,
                                                        int64_t dst_ld, int64_t dst_bstride,
                                                        int64_t col0) {
  constexpr int EPC = TileOf<E>::EPC, CPR = TileOf<E>::CPR;
  __shared__ __attribute__((aligned(16))) E tile[64][TileOf<E>::P];
  const int64_t b = blockIdx.z;
  if (active && active[b] == 0) return;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 64, r0 = static_cast<int64_t>(blockIdx.y) * 64;
  const E *s = src + b * R * C;
  for (int i = threadIdx.x; i < 64 * CPR; i += 256) {
    const int r = i / CPR, cc = i % CPR;
    if (r0 + r < R && c0 + EPC * cc < C)
      *reinterpret_cast<uint4 *>(&tile[r][TileOf<E>::col(r, EPC * cc)]) =
          *reinterpret_cast<const uint4 *>(s + (r0 + r) * C + c0 + EPC * cc);
  }
  __syncthreads();
  tile_store_cols<E>(tile, c0, C, r0, R, dst + b * dst_bstride + col0, dst_ld);
}

// Rows of a matrix as columns of dst (ld ldd): destination column q holds
// source row r(q) (read from row_index[r] if given, times row_scale[r] if
// given); dense: r(q) = q, valid below R; grouped: column runs of padded
// length per group, r(q) = off[e] + q - poff[e] for poff[e] <= q < poff[e+1],
// valid below off[e + 1]. Invalid columns (the padding) are written as
// zeros, up to Q columns (grouped: poff[G]).
template <typename E>
__global__ __launch_bounds__(256) void cols_kernel(const E *src, int64_t ld_src,
                                                   const int32_t *row_index,
                                                   const float *row_scale, int64_t R, int64_t C,
                                                   const int32_t *off, const int32_t *poff, int G,
                                                   int64_t Q, E *dst, int64_t ldd) {
  constexpr int EPC = TileOf<E>::EPC, CPR = TileOf<E>::CPR;
  using CK = typename ChunkT<E>::C;
  __shared__ __attribute__((aligned(16))) E tile[64][TileOf<E>::P];
  __shared__ int64_t srow[64];
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 64, q0 = static_cast<int64_t>(blockIdx.y) * 64;
  const int64_t qend = off ? poff[G] : Q;
  if (q0 >= qend) return;
  if (threadIdx.x < 64) {
    const int64_t q = q0 + threadIdx.x;
    int64_t r = -1;
    if (q < qend) {
      if (off) {
        int lo = 0, hi = G;  // group e with poff[e] <= q < poff[e + 1]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (poff[mid] <= q) lo = mid; else hi = mid;
        }
        const int64_t rr = off[lo] + (q - poff[lo]);
        r = rr < off[lo + 1] ? rr : -1;
      } else {
        r = q < R ? q : -1;
      }
    }
    srow[threadIdx.x] = r;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * CPR; i += 256) {
    const int qi = i / CPR, cc = i % CPR;
    if (c0 + EPC * cc >= C) continue;
    const int64_t r = srow[qi];
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r >= 0) {
      const int64_t sr = row_index ? row_index[r] : r;
      v = *reinterpret_cast<const uint4 *>(src + sr * ld_src + c0 + EPC * cc);
      if (row_scale) {
        float f[EPC];
        CK::unpack(v, f);
        const float sc = row_scale[r];
#pragma unroll
        for (int j = 0; j < EPC; ++j) f[j] *= sc;
        v = CK::pack(f);
      }
    }
    *reinterpret_cast<uint4 *>(&tile[qi][TileOf<E>::col(qi, EPC * cc)]) = v;
  }
  __syncthreads();
  tile_store_cols<E>(tile, c0, C, q0, qend, dst, ldd);
}

// Padded expert column offsets poff[e] = sum of round64(counts) before e, and
// the K-grouped m-tile table of each output height M (bm rows per tile): one
// run of ceil(M / bm) tiles per active expert, grouped per expert.
__global__ __launch_bounds__(1024) void kgroup_kernel(const int32_t *counts, int E, int M1, int M2,
                                                      int bm, int32_t *poff, int32_t *t1,
                                                      int32_t *n1, int32_t *t2, int32_t *n2) {
  __shared__ int tmp[1024];
  const int t = threadIdx.x;
  const int c = t < E ? counts[t] : 0;
  int total;
  const int ex = block_exscan_1024((c + 63) / 64 * 64, tmp, &total);
  if (t < E) poff[t] = ex;
  if (t == 0) poff[E] = total;
  for (int w = 0; w < 2; ++w) {
    const int M = w ? M2 : M1;
    int32_t *tab = w ? t2 : t1;
    const int per = (M + bm - 1) / bm;
    int ntot;
    const int start = block_exscan_1024(c > 0 ? per : 0, tmp, &ntot);
    if (t < E && c > 0) {
      for (int i = 0; i < per; ++i) {
        int32_t *ti = tab + kTileInts * static_cast<int64_t>(start + i);
        ti[0] = t;
        ti[1] = i * bm;
        ti[2] = min((i + 1) * bm, M);
        ti[3] = start + i / kTileGroup * kTileGroup;
        ti[4] = min(kTileGroup, per - i / kTileGroup * kTileGroup);
      }
    }
    if (t == 0) *(w ? n2 : n1) = ntot;
    __syncthreads();
  }
}

// Per row p (one wavefront): from the pre-activations a, u and the unscaled
// W_down^T dy (fp32 [R, f]) and the routing weight g[p] (1 if null): h =
// SiLU(a) u, dh = g W_down^T dy, da = dh u SiLU'(a), du = dh SiLU(a) in the
// activation type (dAU row p = [da | du], 2 f wide), and dg[p] = <W_down^T dy, h> (if dg).
template <typename AT>
__global__ __launch_bounds__(256) void rows_kernel(const float *A, const float *U, const float *D,
                                                   const float *gw, int64_t R, int f, void *H,
                                                   void *dAU, float *dg) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (p >= R) return;
  const int lane = threadIdx.x & 63;
  const float g = gw ? gw[p] : 1.0f;
  float acc = 0.f;
  const int64_t o = p * f;
  if (!D) {  // h only (a forward recompute)
    for (int j = lane; j < f; j += 64) {
      const float a = A[o + j];
      Elem<AT>::store(H, o + j, a / (1.0f + expf(-a)) * U[o + j]);
    }
    return;
  }
  for (int j = lane; j < f; j += 64) {
    const float a = A[o + j], u = U[o + j], dd = D[o + j];
    const float s = 1.0f / (1.0f + expf(-a));
    const float si = a * s;
    const float h = si * u;
    acc += dd * h;
    const float dh = g * dd;
    Elem<AT>::store(H, o + j, h);
    Elem<AT>::store(dAU, 2 * o + j, dh * u * s * (1.0f + a * (1.0f - s)));
    Elem<AT>::store(dAU, 2 * o + f + j, dh * si);
  }
  if (dg) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) dg[p] = acc;
  }
}

// dx[t] = sum_k dXs[inv[t K + k]] + add1[t] + add2[t]
//         + sum_k dr[inv[t K + k]] W_router[idx[t K + k]]
// (each term optional; fp32, k in order, then stored in the activation type);
// one wavefront per token and 256-column block (blockIdx.y).
template <typename AT>
__global__ __launch_bounds__(256) void dx_kernel(const float *dXs, const float *dXsh,
                                                 const float *add2, const int32_t *inv,
                                                 const int32_t *idx, const float *dr,
                                                 const float *wr, int64_t T, int K, int d,
                                                 void *dx) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int i = blockIdx.y * 256 + (threadIdx.x & 63) * 4;
  if (t >= T || i >= d) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (dXs) {
    for (int k = 0; k < K; ++k) {
      const int64_t q = inv[t * K + k];
      const float4 v = *reinterpret_cast<const float4 *>(dXs + q * d + i);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
  }
  if (dXsh) {
    const float4 v = *reinterpret_cast<const float4 *>(dXsh + t * d + i);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  if (add2) {
    const float4 v = *reinterpret_cast<const float4 *>(add2 + t * d + i);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  if (dr) {
    for (int k = 0; k < K; ++k) {
      const float c = dr[inv[t * K + k]];
      const float4 w = *reinterpret_cast<const float4 *>(wr + static_cast<int64_t>(idx[t * K + k]) * d + i);
      acc.x += c * w.x; acc.y += c * w.y; acc.z += c * w.z; acc.w += c * w.w;
    }
  }
  Elem<AT>::store(dx, t * d + i, acc.x);
  Elem<AT>::store(dx, t * d + i + 1, acc.y);
  Elem<AT>::store(dx, t * d + i + 2, acc.z);
  Elem<AT>::store(dx, t * d + i + 3, acc.w);
}

// dW_router[e, i] = sum over the rows p of expert e (sorted order) of
// dr[p] x[sorted_token[p], i], fp32. Block (column block, e, z) of Z sums the
// rows offsets[e] + z + j Z (j = 0, 1, ...) in order, one thread per column,
// into part[e, z, i] (Z > 1) or straight into dwr (Z == 1); dwr_final_kernel
// adds the Z partials in order.
template <typename AT>
__global__ __launch_bounds__(256) void dwr_kernel(const float *dr, const int32_t *stok,
                                                  const int32_t *offsets, const void *x, int d,
                                                  int Z, float *part, float *dwr) {
  const int e = blockIdx.y, z = blockIdx.z;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= d) return;
  const int p0 = offsets[e] + z, p1 = offsets[e + 1];
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;  // rows j = 0, 1, 2, 3 mod 4
  int p = p0;
  for (; p + 3 * Z < p1; p += 4 * Z) {
    const int64_t r0 = stok[p], r1 = stok[p + Z], r2 = stok[p + 2 * Z], r3 = stok[p + 3 * Z];
    a0 += dr[p] * Elem<AT>::load(x, r0 * d + i);
    a1 += dr[p + Z] * Elem<AT>::load(x, r1 * d + i);
    a2 += dr[p + 2 * Z] * Elem<AT>::load(x, r2 * d + i);
    a3 += dr[p + 3 * Z] * Elem<AT>::load(x, r3 * d + i);
  }
  for (; p < p1; p += Z) a0 += dr[p] * Elem<AT>::load(x, static_cast<int64_t>(stok[p]) * d + i);
  const float acc = (a0 + a1) + (a2 + a3);
  if (Z == 1)
    dwr[static_cast<int64_t>(e) * d + i] = acc;
  else
    part[(static_cast<int64_t>(e) * Z + z) * d + i] = acc;
}

__global__ __launch_bounds__(256) void dwr_final_kernel(const float *part, int d, int Z,
                                                        float *dwr) {
  const int e = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= d) return;
  float acc = 0.f;
  for (int z = 0; z < Z; ++z) acc += part[(static_cast<int64_t>(e) * Z + z) * d + i];
  dwr[static_cast<int64_t>(e) * d + i] = acc;
}

// Latent layer ("StableLatentMoE and QuantileBalancer", "Return to model
// width"), one wavefront per token. Forward recompute: R = sum_k Y[inv[t K +
// k]] (fp32, k in order), rinv = 1 / sqrt(mean(R^2) + eps) (1 without the
// norm), R' = R rinv gamma in the activation type (gamma = 1 if null).
template <typename AT>
__global__ __launch_bounds__(256) void latent_fwd_kernel(const float *Y, const int32_t *inv,
                                                         int64_t T, int K, int L, int norm,
                                                         float eps, const float *gamma, float *R,
                                                         float *rinv, void *Rp) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  float ss = 0.f;
  for (int l = lane; l < L; l += 64) {
    float v = 0.f;
    for (int k = 0; k < K; ++k) v += Y[static_cast<int64_t>(inv[t * K + k]) * L + l];
    R[t * L + l] = v;
    ss += v * v;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const float r = norm ? 1.0f / sqrtf(ss / static_cast<float>(L) + eps) : 1.0f;
  if (lane == 0) rinv[t] = r;
  for (int l = lane; l < L; l += 64) {
    const float gm = (norm && gamma) ? gamma[l] : 1.0f;
    Elem<AT>::store(Rp, t * L + l, R[t * L + l] * r * gm);
  }
}

// RMSNorm backward per token: s = gamma dR' (dR' = W_lat_up^T dy, fp32),
// dR = rinv s - R rinv^3 <s, R> / L (dR = dR' without the norm), in the
// activation type.
template <typename AT>
__global__ __launch_bounds__(256) void latent_bwd_kernel(const float *dRp, const float *R,
                                                         const float *rinv, const float *gamma,
                                                         int64_t T, int L, int norm, void *dR) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const int64_t o = t * L;
  if (!norm) {
    for (int l = lane; l < L; l += 64) Elem<AT>::store(dR, o + l, dRp[o + l]);
    return;
  }
  float sR = 0.f;
  for (int l = lane; l < L; l += 64) sR += dRp[o + l] * (gamma ? gamma[l] : 1.0f) * R[o + l];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sR += __shfl_xor(sR, off);
  const float r = rinv[t];
  const float c = r * r * r * sR / static_cast<float>(L);
  for (int l = lane; l < L; l += 64)
    Elem<AT>::store(dR, o + l, r * dRp[o + l] * (gamma ? gamma[l] : 1.0f) - R[o + l] * c);
}

// Column sums sum_t A[t, l] B[t, l] s[t] in two passes (fixed order): per
// block of 256 tokens into part[blk, l], then the blocks in order.
__global__ __launch_bounds__(256) void colsum_part_kernel(const float *A, const float *B,
                                                          const float *sc, int64_t T, int L,
                                                          float *part) {
  const int l = blockIdx.x * 256 + threadIdx.x;
  if (l >= L) return;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * 256;
  const int64_t t1 = t0 + 256 < T ? t0 + 256 : T;
  float acc = 0.f;
  for (int64_t t = t0; t < t1; ++t) acc += A[t * L + l] * B[t * L + l] * sc[t];
  part[static_cast<int64_t>(blockIdx.y) * L + l] = acc;
}

__global__ __launch_bounds__(256) void colsum_final_kernel(const float *part, int64_t nblk, int L,
                                                           float *out) {
  const int l = blockIdx.x * 256 + threadIdx.x;
  if (l >= L) return;
  float acc = 0.f;
  for (int64_t b = 0; b < nblk; ++b) acc += part[b * L + l];
  out[l] = acc;
}

}  // namespace

hipError_t launch_fill0(void *p, size_t bytes, hipStream_t s) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  if (n16 == 0) return hipSuccess;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  fill0_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(static_cast<uint4 *>(p), n16);
  return hipGetLastError();
}

hipError_t launch_transpose(const void *src, int64_t batches, int64_t R, int64_t C,
                            const int32_t *active, void *dst, int64_t dst_ld, int64_t dst_bstride,
                            int64_t col0, int act_bf16, hipStream_t s) {
  if (batches == 0 || R == 0 || C == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>((C + 63) / 64), static_cast<unsigned>((R + 63) / 64),
            static_cast<unsigned>(batches));
  if (act_bf16)
    transpose_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t *>(src), R, C,
                                                    active, static_cast<uint16_t *>(dst), dst_ld,
                                                    dst_bstride, col0);
  else
    transpose_kernel<uint32_t><<<grid, 256, 0, s>>>(static_cast<const uint32_t *>(src), R, C,
                                                    active, static_cast<uint32_t *>(dst), dst_ld,
                                                    dst_bstride, col0);
  return hipGetLastError();
}

hipError_t launch_cols(const void *src, int64_t ld_src, const int32_t *row_index,
                       const float *row_scale, int64_t R, int64_t C, const int32_t *off,
                       const int32_t *poff, int G, int64_t Q, void *dst, int64_t ldd,
                       int act_bf16, hipStream_t s) {
  if (Q == 0 || C == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>((C + 63) / 64), static_cast<unsigned>((Q + 63) / 64));
  if (act_bf16)
    cols_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t *>(src), ld_src,
                                               row_index, row_scale, R, C, off, poff, G, Q,
                                               static_cast<uint16_t *>(dst), ldd);
  else
    cols_kernel<uint32_t><<<grid, 256, 0, s>>>(static_cast<const uint32_t *>(src), ld_src,
                                               row_index, row_scale, R, C, off, poff, G, Q,
                                               static_cast<uint32_t *>(dst), ldd);
  return hipGetLastError();
}

hipError_t launch_kgroup(const int32_t *counts, int E, int M1, int M2, int bm, int32_t *poff,
                         int32_t *t1, int32_t *n1, int32_t *t2, int32_t *n2, hipStream_t s) {
  kgroup_kernel<<<1, 1024, 0, s>>>(counts, E, M1, M2, bm, poff, t1, n1, t2, n2);
  return hipGetLastError();
}

hipError_t launch_bwd_rows(const float *A, const float *U, const float *D, const float *gw,
                           int64_t R, int f, void *H, void *dAU, float *dg, int act_bf16,
                           hipStream_t s) {
  if (R == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>((R + 3) / 4);
  if (act_bf16)
    rows_kernel<bf16_t><<<grid, 256, 0, s>>>(A, U, D, gw, R, f, H, dAU, dg);
  else
    rows_kernel<float><<<grid, 256, 0, s>>>(A, U, D, gw, R, f, H, dAU, dg);
  return hipGetLastError();
}

hipError_t launch_bwd_dx(const float *dXs, const float *dXsh, const float *add2,
                         const int32_t *inv, const int32_t *idx, const float *dr, const float *wr,
                         int64_t T, int K, int d, void *dx, int act_bf16, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((T + 3) / 4), static_cast<unsigned>((d + 255) / 256));
  if (act_bf16)
    dx_kernel<bf16_t><<<grid, 256, 0, s>>>(dXs, dXsh, add2, inv, idx, dr, wr, T, K, d, dx);
  else
    dx_kernel<float><<<grid, 256, 0, s>>>(dXs, dXsh, add2, inv, idx, dr, wr, T, K, d, dx);
  return hipGetLastError();
}

int dwr_splits(int E, int d) {
  const int blocks = E * ((d + 255) / 256);
  const int z = (4096 + blocks - 1) / blocks;
  return z < 1 ? 1 : (z > 64 ? 64 : z);
}

size_t dwr_part_bytes(int E, int d) {
  const int z = dwr_splits(E, d);
  return z > 1 ? static_cast<size_t>(E) * z * d * 4 : 0;
}

hipError_t launch_bwd_dwr(const float *dr, const int32_t *stok, const int32_t *offsets,
                          const void *x, int E, int d, float *part, float *dwr, int act_bf16,
                          hipStream_t s) {
  if (E == 0 || d == 0) return hipSuccess;
  const int Z = dwr_splits(E, d);
  const dim3 grid(static_cast<unsigned>((d + 255) / 256), static_cast<unsigned>(E),
                  static_cast<unsigned>(Z));
  if (act_bf16)
    dwr_kernel<bf16_t><<<grid, 256, 0, s>>>(dr, stok, offsets, x, d, Z, part, dwr);
  else
    dwr_kernel<float><<<grid, 256, 0, s>>>(dr, stok, offsets, x, d, Z, part, dwr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || Z == 1) return e;
  dwr_final_kernel<<<dim3(static_cast<unsigned>((d + 255) / 256), static_cast<unsigned>(E)), 256,
                     0, s>>>(part, d, Z, dwr);
  return hipGetLastError();
}

hipError_t launch_latent_fwd(const float *Y, const int32_t *inv, int64_t T, int K, int L,
                             int norm, float eps, const float *gamma, float *R, float *rinv,
                             void *Rp, int act_bf16, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>((T + 3) / 4);
  if (act_bf16)
    latent_fwd_kernel<bf16_t><<<grid, 256, 0, s>>>(Y, inv, T, K, L, norm, eps, gamma, R, rinv, Rp);
  else
    latent_fwd_kernel<float><<<grid, 256, 0, s>>>(Y, inv, T, K, L, norm, eps, gamma, R, rinv, Rp);
  return hipGetLastError();
}

hipError_t launch_latent_bwd(const float *dRp, const float *R, const float *rinv,
                             const float *gamma, int64_t T, int L, int norm, void *dR,
                             int act_bf16, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>((T + 3) / 4);
  if (act_bf16)
    latent_bwd_kernel<bf16_t><<<grid, 256, 0, s>>>(dRp, R, rinv, gamma, T, L, norm, dR);
  else
    latent_bwd_kernel<float><<<grid, 256, 0, s>>>(dRp, R, rinv, gamma, T, L, norm, dR);
  return hipGetLastError();
}

int64_t colsum_blocks(int64_t T) { return (T + 255) / 256; }

hipError_t launch_colsum(const float *A, const float *B, const float *sc, int64_t T, int L,
                         float *part, float *out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 g1(static_cast<unsigned>((L + 255) / 256), static_cast<unsigned>(colsum_blocks(T)));
  colsum_part_kernel<<<g1, 256, 0, s>>>(A, B, sc, T, L, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  colsum_final_kernel<<<static_cast<unsigned>((L + 255) / 256), 256, 0, s>>>(
      part, colsum_blocks(T), L, out);
  return hipGetLastError();
}

}  // namespace moe
