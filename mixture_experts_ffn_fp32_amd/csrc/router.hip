// Router: fp32 logits, top-(K+1) selection and routing weights.
//
// APEX-1 Mathematical Reference - Part 3, section 13.2: r = x W_router + b,
// top-K of r, g = softmax over the K selected. "A working MoE layer in
// PyTorch": softmax over all experts in fp32, top-K, renormalise (the same
// weights in exact arithmetic). "StableLatentMoE and QuantileBalancer": fp32
// router, sigmoid scores, bias-corrected top-(K+1), last candidate dropped,
// weights are the uncorrected sigmoid scores.
//
// Logits (fp32 router on matrix cores). For bf16 activations, each fp32
// router weight w is split exactly into three bf16 values, w = h + m + l
// (h = bf16(w), m = bf16(w - h), l = w - h - m, which fits in bf16 because
// 24 significand bits = 3 x 8). A bf16 x times a bf16 plane is exact in
// fp32, so x W^T = x H^T + x M^T + x L^T is the fp32 router product computed
// on v_mfma_f32_16x16x32_bf16 with fp32 accumulation: one GEMM against the
// stacked planes [H; M; L] gives three partial logits per expert, summed
// (h + m) + l in the selection kernel. For fp32 activations the GEMM runs on
// v_mfma_f32_16x16x4_f32 directly. Either way the accumulation rounds once
// per 32 (bf16) or 4 (fp32) products instead of once per product.
//
// Selection: one wavefront per token. Each lane holds E/64 scores. Up to 64
// experts, every lane ranks its expert against all the others at once;
// otherwise K+1 rounds of a (value, lower id) max-reduction over the 64
// lanes (DPP moves inside rows of 16 lanes, readlane across the rows) pick
// the experts in descending order. Ties go to the lower id either way.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kMaxK = 16;
constexpr int kMaxE = 1024;
constexpr int kPerLane = kMaxE / 64;
// one-wavefront-per-token router: at most 64 experts and this model width
constexpr int kValuMaxE = 64;
constexpr int kValuMaxD = 2048;

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }

// Logit of expert e from the partials of token row lg ([splits][T, parts*E]
// with split stride ss): each plane's K-split partials summed in split
// order, then the planes high + mid + low. Every consumer of the logits
// calls this, so they all see the same fp32 value.
// (All of a logit's partials are loaded before they are added, split by
// split in order: at most kMaxRouterSplits splits.)
constexpr int kMaxRouterSplits = 8;
__device__ __forceinline__ float logit_of(const float *lg, int e, int E, int parts, int splits,
                                          int64_t ss) {
  float v[3][kMaxRouterSplits];
#pragma unroll
  for (int q = 0; q < kMaxRouterSplits; ++q) {
    const float *ls = lg + q * ss;
    const bool on = q < splits;
    v[0][q] = on ? ls[e] : 0.f;
    v[1][q] = on && parts == 3 ? ls[E + e] : 0.f;
    v[2][q] = on && parts == 3 ? ls[2 * E + e] : 0.f;
  }
  float pl[3] = {0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < kMaxRouterSplits; ++q)
    if (q < splits) {
      pl[0] += v[0][q];
      pl[1] += v[1][q];
      pl[2] += v[2][q];
    }
  return parts == 3 ? (pl[0] + pl[1]) + pl[2] : pl[0];
}

// planes[0..2][i] = exact bf16 split of w[i]
__global__ __launch_bounds__(256) void split_kernel(const float *__restrict__ w, int64_t n,
                                                    uint16_t *__restrict__ planes) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const float v = w[i];
    const uint16_t h = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(h);
    const uint16_t m = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(m);
    planes[i] = h;
    planes[n + i] = m;
    planes[2 * n + i] = f32_to_bf16(r2);
  }
}

// Wavefront maximum of a 64-bit key, returned to every lane: inside each row
// of 16 lanes by DPP moves (swaps within quads, then the half-row and the
// row mirror, each pairing a lane with one whose partial maximum covers the
// lanes it lacks), then the four row maxima through readlane.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t k) {
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(k)), CTRL, 0xF, 0xF,
                                  false));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(k >> 32)), CTRL, 0xF,
                                  0xF, false));
  const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
  return o > k ? o : k;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t k, int l) {
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(k)), l));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(k >> 32)), l));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
  k = dpp_max_u64<0xB1>(k);   // quad_perm [1, 0, 3, 2]
  k = dpp_max_u64<0x4E>(k);   // quad_perm [2, 3, 0, 1]
  k = dpp_max_u64<0x141>(k);  // row_half_mirror
  k = dpp_max_u64<0x140>(k);  // row_mirror
  const uint64_t r0 = readlane_u64(k, 0), r1 = readlane_u64(k, 16);
  const uint64_t r2 = readlane_u64(k, 32), r3 = readlane_u64(k, 48);
  const uint64_t a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
  return a > b ? a : b;
}

// Wavefront sum of one float per lane, the same in every lane: DPP adds
// inside each row of 16 lanes (the pairings of wave_max_u64), then the four
// row sums, (row 0 + row 1) + (row 2 + row 3). A fixed order: the result
// depends only on the 64 inputs.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Ranking key of (score, expert id): larger score first, then lower id. The
// score's bits are mapped to an unsigned order (negative values inverted)
// after -0 is made +0, so equal scores compare equal as floats do.
__device__ __forceinline__ uint64_t rank_key(float v, int id) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  const uint32_t o = (u >> 31) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(o) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(id));
}

// Selection of token t by one wavefront from its logits: lane l holds the
// logits of experts l + 64 j (j < PL, PL * 64 >= E) in raw[j]. Writes idx, g
// and the optional gap / top scores.
template <int PL>
__device__ __forceinline__ void select_from(const RouterArgs &a, int64_t t, int lane,
                                            const float (&raw)[PL]) {
  const int E = a.E, K = a.K;
  const int nsel = K + 1 <= E ? K + 1 : E;
  const bool sig = a.mode == 2;
  float v[PL];  // ranking score
  float vmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    const int e = lane + 64 * j;
    float sc = -INFINITY;
    if (e < E) {
      const float b = a.bias ? a.bias[e] : 0.f;
      sc = sig ? sigmoidf_(raw[j]) + b : raw[j] + b;
      vmax = fmaxf(vmax, sc);
    }
    v[j] = sc;
  }
  // the softmax-first rule reports probabilities: all-expert normaliser
  float zall = 1.f;
  if (a.mode == 1) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, off));
    zall = 0.f;
#pragma unroll
    for (int j = 0; j < PL; ++j)
      if (lane + 64 * j < E) zall += expf(v[j] - vmax);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) zall += __shfl_xor(zall, off);
  }

  if constexpr (PL == 1) {
    // at most 64 experts, one per lane: each lane's rank among them, counted
    // against every other lane's key (the same order as the rounds below:
    // larger score first, ties to the lower id); rank r < K is slot r.
    // Lanes without an expert hold key 0 and rank 64.
    const bool valid = lane < E;
    const uint64_t key = valid ? rank_key(v[0], lane) : 0;
    int rk[4] = {0, 0, 0, 0};
    const int e4 = (E + 3) & ~3;
    for (int l0 = 0; l0 < e4; l0 += 4) {
#pragma unroll
      for (int q = 0; q < 4; ++q) rk[q] += readlane_u64(key, l0 + q) > key ? 1 : 0;
    }
    const int rank = valid ? (rk[0] + rk[1]) + (rk[2] + rk[3]) : 64;
    auto lane_of = [&](int r) {  // the lane holding rank r (uniform)
      const uint64_t b = __ballot(rank == r);
      return b ? static_cast<int>(__builtin_ctzll(b)) : 0;
    };
    auto at = [&](float x, int l) {
      return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
    };
    const bool chosen = rank < K;
    const float top0 = at(v[0], lane_of(0));  // the largest ranking score
    const float w = !chosen ? 0.f : (sig ? sigmoidf_(raw[0]) : expf(v[0] - top0));
    const float z = wave_sum_f32(w);
    const float gw = (sig && !a.renormalize) ? w : w / z;
    if (chosen) {
      a.idx[t * K + rank] = lane;
      a.g[t * K + rank] = gw * a.routed_scale;
    }
    // scores in the ranked space
    const float rsv = a.mode == 1 ? expf(v[0] - vmax) / zall : v[0];
    if (a.gap) {
      const float gp = K < E ? at(rsv, lane_of(K - 1)) - at(rsv, lane_of(K)) : INFINITY;
      if (lane == 0) a.gap[t] = gp;
    }
    if (a.top) {
      if (rank <= K) a.top[t * (K + 1) + rank] = rsv;
      if (K >= E && lane == 0) a.top[t * (K + 1) + K] = -INFINITY;  // no expert of rank K
    }
    return;
  }

  float sv[kMaxK + 1], sraw[kMaxK + 1];
  int si[kMaxK + 1];
#pragma unroll
  for (int r = 0; r <= kMaxK; ++r) {
    sv[r] = -INFINITY;
    sraw[r] = 0.f;
    si[r] = 0;
    if (r < nsel) {
      float bv = -INFINITY, br = 0.f;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int j = 0; j < PL; ++j)
        if (v[j] > bv) {  // ids ascend within a lane: ties keep the lower id
          bv = v[j];
          br = raw[j];
          bi = lane + 64 * j;
        }
      // the winner's lane holds its score and logit as its own best
      const uint64_t win = wave_max_u64(rank_key(bv, bi));
      bi = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(win));
      const int wl = __builtin_amdgcn_readfirstlane(bi & 63);
      sv[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), wl));
      sraw[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(br), wl));
      si[r] = bi;
#pragma unroll
      for (int j = 0; j < PL; ++j)
        if (lane + 64 * j == bi) v[j] = -INFINITY;
    }
  }
  // the selection is the same in every lane: each lane computes the weights
  // and stores its own slot (lane k < K: idx and g of slot k, lane r <= K:
  // the r-th top score), so a token's stores are one instruction each
  float gk[kMaxK];
  float z = 0.f;
  if (sig) {
#pragma unroll
    for (int k = 0; k < kMaxK; ++k)
      if (k < K) {
        gk[k] = sigmoidf_(sraw[k]);
        z += gk[k];
      }
    if (a.renormalize) {
#pragma unroll
      for (int k = 0; k < kMaxK; ++k)
        if (k < K) gk[k] = gk[k] / z;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kMaxK; ++k)
      if (k < K) {
        gk[k] = expf(sv[k] - sv[0]);
        z += gk[k];
      }
#pragma unroll
    for (int k = 0; k < kMaxK; ++k)
      if (k < K) gk[k] = gk[k] / z;
  }
  int my_i = 0;
  float my_g = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxK; ++k)
    if (k < K && lane == k) {
      my_i = si[k];
      my_g = gk[k];
    }
  if (lane < K) {
    a.idx[t * K + lane] = my_i;
    a.g[t * K + lane] = my_g * a.routed_scale;
  }
  float rs[kMaxK + 1];  // scores in the ranked space
#pragma unroll
  for (int r = 0; r <= kMaxK; ++r)
    rs[r] = (a.mode == 1 && r < nsel) ? expf(sv[r] - vmax) / zall : sv[r];
  if (a.gap && lane == 0) {
    float gp = INFINITY;
#pragma unroll
    for (int r = 1; r <= kMaxK; ++r)
      if (r == K && K < E) gp = rs[r - 1] - rs[r];
    a.gap[t] = gp;
  }
  if (a.top) {
    float my_top = -INFINITY;
#pragma unroll
    for (int r = 0; r <= kMaxK; ++r)
      if (r <= K && lane == r) my_top = r < nsel ? rs[r] : -INFINITY;
    if (lane <= K) a.top[t * (K + 1) + lane] = my_top;
  }
}

// One wavefront per token over the partial logits [splits][T, parts * E]:
// the K-split partials of each plane are summed in split order, then the
// planes high + mid + low.
template <int PL>
__global__ __launch_bounds__(256) void select_kernel(RouterArgs a, int parts, int splits,
                                                     int64_t split_stride) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int lane = threadIdx.x & 63;
  const float *lg = a.logits + t * static_cast<int64_t>(parts) * a.E;
  float raw[PL];
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    const int e = lane + 64 * j;
    raw[j] = e < a.E ? logit_of(lg, e, a.E, parts, splits, split_stride) : 0.f;
  }
  select_from<PL>(a, t, lane, raw);
}

// Router for few experts and a narrow model, one wavefront per token: lane l
// holds elements [512 c + 8 l, 512 c + 8 l + 8) of x for every 512-column
// chunk c; per expert its fp32 partial dot product (fused multiply-adds in
// column order) is summed over the 64 lanes in a fixed order (wave_sum_f32), so
// every lane holds the logit; the logits go to a.logits [T, E] (one plane,
// one split) and, if `select`, straight into the selection.
template <typename T>
__global__ __launch_bounds__(256) void router_valu_kernel(RouterArgs a, int select) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int lane = threadIdx.x & 63;
  constexpr int kMaxChunks = kValuMaxD / 512;
  float xv[kMaxChunks][8];
  const int chunks = (a.d + 511) / 512;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int i0 = 512 * c + 8 * lane;  // d is a multiple of 8: a lane's 8 are all in or out
    const bool in = c < chunks && i0 < a.d;
#pragma unroll
    for (int h = 0; h < 8 / Chunk<T>::N; ++h) {
      uint4 raw4 = make_uint4(0u, 0u, 0u, 0u);
      if (in)
        raw4 = *reinterpret_cast<const uint4 *>(static_cast<const char *>(a.x) +
                                                (t * a.d + i0) * sizeof(T) + 16 * h);
      Chunk<T>::unpack(raw4, &xv[c][h * Chunk<T>::N]);
    }
  }
  // four experts per pass: all their W_router loads are issued before the
  // FMAs (lanes past d read element 0 and add it times x = 0); per expert the
  // sum runs over the chunks in order, then a fixed-order sum over the lanes
  float raw = 0.f;  // logit of expert `lane`
  for (int e0 = 0; e0 < a.E; e0 += 4) {
    float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      if (c < chunks) {
        const int i0 = 512 * c + 8 * lane;
        const int ii = i0 < a.d ? i0 : 0;
        float4 w0[4], w1[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = e0 + j < a.E ? e0 + j : a.E - 1;
          const float *w = a.w + static_cast<int64_t>(e) * a.d + ii;
          w0[j] = *reinterpret_cast<const float4 *>(w);
          w1[j] = *reinterpret_cast<const float4 *>(w + 4);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[j] = fmaf(xv[c][0], w0[j].x, p[j]);
          p[j] = fmaf(xv[c][1], w0[j].y, p[j]);
          p[j] = fmaf(xv[c][2], w0[j].z, p[j]);
          p[j] = fmaf(xv[c][3], w0[j].w, p[j]);
          p[j] = fmaf(xv[c][4], w1[j].x, p[j]);
          p[j] = fmaf(xv[c][5], w1[j].y, p[j]);
          p[j] = fmaf(xv[c][6], w1[j].z, p[j]);
          p[j] = fmaf(xv[c][7], w1[j].w, p[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = wave_sum_f32(p[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane == e0 + j) raw = p[j];
  }
  if (lane < a.E) a.logits[t * a.E + lane] = raw;
  if (select) {
    const float r1[1] = {raw};
    select_from<1>(a, t, lane, r1);
  }
}

// ------------------------------------------------------------ backward
// Router gradient of one token (one wavefront, lane k < K for slot k): from
// the gradients dg of its routing weights (stored per sorted row, found
// through inv) to the gradients dr of its selected logits, written per
// sorted row. With c = routed_scale:
//  - softmax over the selected (and the softmax-first rule, the same function
//    of the selected logits): q = softmax(logits + bias) over the selected,
//    g = c q, dr_k = q_k (c dg_k - sum_j q_j c dg_j);
//  - sigmoid rule: s = sigmoid(logit), g = c s (or c s / sum s when
//    renormalised), dr_k = ds_k s_k (1 - s_k).
__global__ __launch_bounds__(256) void route_bwd_kernel(RouterArgs a, int parts, int splits,
                                                        int64_t ss, const int32_t *inv,
                                                        const float *dg, float *dr) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int lane = threadIdx.x & 63;
  const bool on = lane < a.K;
  int e = 0;
  int64_t p = 0;
  float l = 0.f, g = 0.f;
  if (on) {
    e = a.idx[t * a.K + lane];
    p = inv[t * a.K + lane];
    g = dg[p];
    l = logit_of(a.logits + t * static_cast<int64_t>(parts) * a.E, e, a.E, parts, splits, ss);
  }
  const float c = a.routed_scale;
  float out;
  if (a.mode == 2) {
    const float sg = on ? sigmoidf_(l) : 0.f;
    float S = sg, sdg = g * sg;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      S += __shfl_xor(S, off);
      sdg += __shfl_xor(sdg, off);
    }
    const float ds = a.renormalize ? c * (g / S - sdg / (S * S)) : c * g;
    out = ds * sg * (1.0f - sg);
  } else {
    const float z = on ? l + (a.bias ? a.bias[e] : 0.f) : -INFINITY;
    float m = z;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    const float ex = on ? expf(z - m) : 0.f;
    float Z = ex;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) Z += __shfl_xor(Z, off);
    const float q = ex / Z;
    float qdg = q * c * g;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) qdg += __shfl_xor(qdg, off);
    out = q * (c * g - qdg);
  }
  if (on) dr[p] = out;
}

// ------------------------------------------------------------ QuantileBalancer
// d[e][t] = thresh_t - sigmoid(logit[t, e]), thresh_t = the token's (K+1)-th
// corrected score (top[t, K]). 64 tokens x 64 experts per workgroup,
// transposed through LDS so both the logit reads and the writes coalesce.
__global__ __launch_bounds__(256) void qb_diff_kernel(const float *logits, int parts, int splits,
                                                      int64_t ss, const float *top, int64_t T,
                                                      int E, int K, float *d) {
  __shared__ float tile[64][65];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int e0 = blockIdx.y * 64;
  const int lx = threadIdx.x & 63, ly = threadIdx.x >> 6;  // 4 rows per pass
  const int64_t rowlen = static_cast<int64_t>(parts) * E;
  for (int r = ly; r < 64; r += 4) {
    const int64_t t = t0 + r;
    const int e = e0 + lx;
    if (t < T && e < E) {
      const float l = logit_of(logits + t * rowlen, e, E, parts, splits, ss);
      tile[r][lx] = top[t * (K + 1) + K] - sigmoidf_(l);
    }
  }
  __syncthreads();
  for (int r = ly; r < 64; r += 4) {
    const int e = e0 + r;
    const int64_t t = t0 + lx;
    if (t < T && e < E) d[static_cast<int64_t>(e) * T + t] = tile[lx][r];
  }
}

// order-preserving map of a finite float to uint32 and back
__device__ __forceinline__ uint32_t ord_of(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_of(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// q[e] = the rank-th smallest of d[e][0..T) (one workgroup per expert):
// four 8-bit radix passes, most significant digit first, each counting the
// candidates that match the digits fixed so far.
__global__ __launch_bounds__(256) void qb_select_kernel(const float *d, int64_t T, int64_t rank,
                                                        float *q) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix, s_rank;
  const int e = blockIdx.x;
  const float *col = d + static_cast<int64_t>(e) * T;
  if (threadIdx.x == 0) {
    s_prefix = 0;
    s_rank = static_cast<uint32_t>(rank);
  }
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    hist[threadIdx.x] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix;
    for (int64_t t = threadIdx.x; t < T; t += 256) {
      const uint32_t k = ord_of(col[t]);
      if ((k & hi_mask) == (prefix & hi_mask)) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x == 0) {  // first digit whose running count passes the rank
      uint32_t acc = 0, r = s_rank;
      int dg = 0;
      for (; dg < 255; ++dg) {
        if (acc + hist[dg] > r) break;
        acc += hist[dg];
      }
      s_rank = r - acc;
      s_prefix = prefix | (static_cast<uint32_t>(dg) << shift);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) q[e] = float_of(s_prefix);
}

// new_bias[e] = q[e] - mean(q), the mean summed in fp64 in expert order
__global__ __launch_bounds__(256) void qb_center_kernel(const float *q, int E, float *new_bias) {
  __shared__ double s_mean;
  if (threadIdx.x == 0) {
    double m = 0.0;
    for (int e = 0; e < E; ++e) m += static_cast<double>(q[e]);
    s_mean = m / E;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    new_bias[e] = static_cast<float>(static_cast<double>(q[e]) - s_mean);
}

// ------------------------------------------------------------ router losses
// Load-balancing (Switch) loss of "A working MoE layer in PyTorch": alpha * E
// * sum_e f_e P_e with f_e = counts[e] / (T K) and P_e the mean over tokens of
// softmax(logits_t)_e; router z-loss of the transformer book's MoE chapter
// (MoEAuxiliaryLoss.router_z_loss): z_weight * mean over tokens of
// logsumexp(logits_t)^2. Both read the router's own logits x W^T (the balance
// bias is a non-gradient nudge and stays out).
//
// Stage 1: one workgroup per chunk of 16 to 64 tokens (a quarter per
// wavefront, in token order; chunks sized so a call has about 256 of them);
// each lane keeps the running softmax sums of the experts it owns; the four
// wavefronts' sums are added in wavefront order. part[chunk] = {P sums [E],
// sum of lse^2}. Stage 2 adds the chunks in chunk order in fp64.
constexpr int kLossMinTokens = 16, kLossMaxTokens = 64, kLossChunks = 256;

template <int PL>
__global__ __launch_bounds__(256) void loss_partial_kernel(const float *logits, int parts,
                                                           int splits, int64_t ss, int64_t T,
                                                           int E, int chunk_tokens, float *part) {
  __shared__ float sh[4][kMaxE + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int per_wave = chunk_tokens / 4;
  const int64_t t_begin = static_cast<int64_t>(blockIdx.x) * chunk_tokens + wave * per_wave;
  float acc[PL];
#pragma unroll
  for (int j = 0; j < PL; ++j) acc[j] = 0.f;
  float zacc = 0.f;
  for (int i = 0; i < per_wave; ++i) {
    const int64_t t = t_begin + i;
    if (t >= T) break;
    const float *lg = logits + t * static_cast<int64_t>(parts) * E;
    float l[PL];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      const int e = lane + 64 * j;
      l[j] = e < E ? logit_of(lg, e, E, parts, splits, ss) : -INFINITY;
      m = fmaxf(m, l[j]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      l[j] = lane + 64 * j < E ? expf(l[j] - m) : 0.f;
      z += l[j];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
    const float rz = 1.0f / z;
#pragma unroll
    for (int j = 0; j < PL; ++j) acc[j] += l[j] * rz;
    const float lse = m + logf(z);
    zacc += lse * lse;
  }
#pragma unroll
  for (int j = 0; j < PL; ++j)
    if (lane + 64 * j < E) sh[wave][lane + 64 * j] = acc[j];
  if (lane == 0) sh[wave][E] = zacc;
  __syncthreads();
  float *out = part + static_cast<int64_t>(blockIdx.x) * (E + 1);
  for (int e = threadIdx.x; e <= E; e += 256)
    out[e] = ((sh[0][e] + sh[1][e]) + sh[2][e]) + sh[3][e];
}

// losses[0] = alpha E sum_e (counts[e] / (T K)) (P_e / T), losses[1] =
// z_weight (sum lse^2) / T; chunk sums in chunk order, expert terms reduced
// in a fixed tree, all in fp64.
__global__ __launch_bounds__(1024) void loss_final_kernel(const float *part, int64_t n_chunks,
                                                          int64_t T, int E, int K,
                                                          const int32_t *counts, float alpha,
                                                          float z_weight, float *losses) {
  // column e of the chunk partials (E + 1 columns: the experts' probability
  // sums, then the z term) is summed in fp64 by J threads, thread j taking
  // chunks j, j + J, ... in order (their loads issued kBatch at a time);
  // then the J sums of each column in order, then the columns by a fixed
  // tree
  constexpr int kBatch = 16;
  __shared__ double ps[kMaxE + 8];
  __shared__ double sa[1024], sz[1024];
  const int t = threadIdx.x, E1 = E + 1;
  const int J = E1 >= 1024 ? 1 : 1024 / E1;
  for (int i = t; i < E1 * J; i += 1024) {
    const int e = i % E1, j = i / E1;
    double s = 0.0;
    for (int64_t c0 = j; c0 < n_chunks; c0 += static_cast<int64_t>(J) * kBatch) {
      float v[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int64_t c = c0 + static_cast<int64_t>(b) * J;
        v[b] = c < n_chunks ? part[c * E1 + e] : 0.f;
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) s += static_cast<double>(v[b]);
    }
    ps[i] = s;
  }
  __syncthreads();
  double a = 0.0, zs = 0.0;
  for (int e = t; e < E1; e += 1024) {
    double s = 0.0;
    for (int j = 0; j < J; ++j) s += ps[j * E1 + e];
    if (e < E)
      a += (static_cast<double>(counts[e]) / (static_cast<double>(T) * K)) * (s / static_cast<double>(T));
    else
      zs = s;
  }
  sa[t] = a;
  sz[t] = zs;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (t < w) {
      sa[t] += sa[t + w];
      sz[t] += sz[t + w];
    }
    __syncthreads();
  }
  if (t == 0) {
    losses[0] = static_cast<float>(static_cast<double>(alpha) * E * sa[0]);
    losses[1] = static_cast<float>(static_cast<double>(z_weight) * sz[0] / static_cast<double>(T));
  }
}

}  // namespace

// Few experts, a narrow model and little work: the one-wavefront-per-token
// router (no weight split, no GEMM launch); else the matrix-core GEMM.
bool router_valu(const RouterArgs &a) {
  return a.E <= kValuMaxE && a.d <= kValuMaxD &&
         a.T * static_cast<int64_t>(a.E) * a.d <= (int64_t(1) << 26);
}

// Layout of the logits the router pass leaves in a.logits: planes x splits.
void logit_layout(const RouterArgs &a, int act_bf16, int *parts, int *splits) {
  if (router_valu(a)) {
    *parts = 1;
    *splits = 1;
  } else {
    *parts = act_bf16 ? 3 : 1;
    *splits = router_splits(a.T, a.d, a.E, act_bf16);
  }
}

hipError_t launch_router_valu(const RouterArgs &a, int act_bf16, int select, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((a.T + 3) / 4);
  if (act_bf16)
    router_valu_kernel<bf16_t><<<blocks, 256, 0, s>>>(a, select);
  else
    router_valu_kernel<float><<<blocks, 256, 0, s>>>(a, select);
  return hipGetLastError();
}

// Router logits only, in the layout logit_layout() reports.
hipError_t launch_router_logits(const RouterArgs &a, int act_bf16, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (router_valu(a)) return launch_router_valu(a, act_bf16, 0, s);
  const int64_t nw = static_cast<int64_t>(a.E) * a.d;
  GemmArgs g{};
  g.a = a.x;
  g.lda = a.d;
  g.ldb = a.d;
  g.K = a.d;
  g.M = a.T;
  g.out = a.logits;
  const int parts = act_bf16 ? 3 : 1;
  g.N = parts * a.E;
  g.ldo = g.N;
  const int splits = router_splits(a.T, a.d, a.E, act_bf16);
  g.k_split = splits;
  g.split_stride = a.T * g.N;
  if (act_bf16) {
    int64_t blocks = (nw + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    split_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(
        a.w, nw, static_cast<uint16_t *>(a.w_split));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    g.b0 = a.w_split;
  } else {
    g.b0 = a.w;
  }
  if (act_bf16 && a.T > 256 && splits > 1 && gemm2_applicable(g, EPI_STORE_F32))
    return launch_gemm2(g, EPI_STORE_F32, TILE2_128x128, s);
  return launch_dense(g, EPI_STORE_F32, act_bf16, s);
}

hipError_t launch_router(const RouterArgs &a, int act_bf16, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (router_valu(a)) return launch_router_valu(a, act_bf16, 1, s);
  hipError_t e = launch_router_logits(a, act_bf16, s);
  if (e != hipSuccess) return e;
  int parts, splits;
  logit_layout(a, act_bf16, &parts, &splits);
  const unsigned blocks = static_cast<unsigned>((a.T + 3) / 4);
  const int64_t ss = a.T * parts * a.E;
  if (a.E <= 64)
    select_kernel<1><<<blocks, 256, 0, s>>>(a, parts, splits, ss);
  else if (a.E <= 256)
    select_kernel<4><<<blocks, 256, 0, s>>>(a, parts, splits, ss);
  else
    select_kernel<kPerLane><<<blocks, 256, 0, s>>>(a, parts, splits, ss);
  return hipGetLastError();
}

// tokens per chunk: a multiple of 4 between 16 and 64, about T / 256
int router_loss_chunk_tokens(int64_t T) {
  int64_t c = (T / kLossChunks + 3) / 4 * 4;
  return static_cast<int>(c < kLossMinTokens ? kLossMinTokens : (c > kLossMaxTokens ? kLossMaxTokens : c));
}

hipError_t launch_router_backward(const RouterArgs &a, int act_bf16, const int32_t *inv,
                                  const float *dg, float *dr, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  int parts, splits;
  logit_layout(a, act_bf16, &parts, &splits);
  route_bwd_kernel<<<static_cast<unsigned>((a.T + 3) / 4), 256, 0, s>>>(
      a, parts, splits, a.T * parts * a.E, inv, dg, dr);
  return hipGetLastError();
}

int64_t router_loss_chunks(int64_t T) {
  const int ct = router_loss_chunk_tokens(T);
  return (T + ct - 1) / ct;
}

hipError_t launch_router_losses(const RouterArgs &a, int act_bf16, const int32_t *counts,
                                float alpha, float z_weight, float *part, float *losses,
                                hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  hipError_t e = launch_router_logits(a, act_bf16, s);
  if (e != hipSuccess) return e;
  int parts, splits;
  logit_layout(a, act_bf16, &parts, &splits);
  const int64_t chunks = router_loss_chunks(a.T);
  const unsigned grid = static_cast<unsigned>(chunks);
  const int ct = router_loss_chunk_tokens(a.T);
  const int64_t ss = a.T * parts * a.E;
  if (a.E <= 64)
    loss_partial_kernel<1><<<grid, 256, 0, s>>>(a.logits, parts, splits, ss, a.T, a.E, ct, part);
  else if (a.E <= 256)
    loss_partial_kernel<4><<<grid, 256, 0, s>>>(a.logits, parts, splits, ss, a.T, a.E, ct, part);
  else
    loss_partial_kernel<kPerLane><<<grid, 256, 0, s>>>(a.logits, parts, splits, ss, a.T, a.E,
                                                       ct, part);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  loss_final_kernel<<<1, 1024, 0, s>>>(part, chunks, a.T, a.E, a.K, counts, alpha, z_weight,
                                       losses);
  return hipGetLastError();
}

hipError_t launch_quantile_balance(const RouterArgs &a, int act_bf16, float *diff, float *q,
                                   float *new_bias, hipStream_t s) {
  if (a.T == 0 || !a.top) return hipErrorInvalidValue;
  hipError_t e = launch_router(a, act_bf16, s);
  if (e != hipSuccess) return e;
  int parts, splits;
  logit_layout(a, act_bf16, &parts, &splits);
  const int64_t ss = a.T * parts * a.E;
  dim3 grid(static_cast<unsigned>((a.T + 63) / 64), static_cast<unsigned>((a.E + 63) / 64));
  qb_diff_kernel<<<grid, 256, 0, s>>>(a.logits, parts, splits, ss, a.top, a.T, a.E, a.K, diff);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // position ceil(p (T - 1)) of the sorted differences, p = K / E, exactly
  const int64_t rank = (static_cast<int64_t>(a.K) * (a.T - 1) + a.E - 1) / a.E;
  qb_select_kernel<<<a.E, 256, 0, s>>>(diff, a.T, rank, q);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  qb_center_kernel<<<1, 256, 0, s>>>(q, a.E, new_bias);
  return hipGetLastError();
}

}  // namespace moe
