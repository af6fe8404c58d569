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
// Selection: one wavefront per token. Each lane holds E/64 scores; K+1
// rounds of a butterfly (value, lower id) max-reduction over the 64 lanes
// pick the experts in descending order, ties to the lower id.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kMaxK = 16;
constexpr int kMaxE = 1024;
constexpr int kPerLane = kMaxE / 64;

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }

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

// One wavefront per token over the partial logits [splits][T, parts * E]:
// the K-split partials of each plane are summed in split order, then the
// planes high + mid + low.
__global__ __launch_bounds__(256) void select_kernel(RouterArgs a, int parts, int splits,
                                                     int64_t split_stride) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int lane = threadIdx.x & 63;
  const int E = a.E, K = a.K;
  const int nsel = K + 1 <= E ? K + 1 : E;
  const bool sig = a.mode == 2;
  const float *lg = a.logits + t * static_cast<int64_t>(parts) * E;

  float raw[kPerLane];  // logit x W^T per owned expert
  float v[kPerLane];    // ranking score
  float vmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) {
    const int e = lane + 64 * j;
    float sc = -INFINITY, l = 0.f;
    if (e < E) {
      float pl[3] = {0.f, 0.f, 0.f};
      for (int q = 0; q < splits; ++q) {
        const float *ls = lg + q * split_stride;
        pl[0] += ls[e];
        if (parts == 3) {
          pl[1] += ls[E + e];
          pl[2] += ls[2 * E + e];
        }
      }
      l = parts == 3 ? (pl[0] + pl[1]) + pl[2] : pl[0];
      const float b = a.bias ? a.bias[e] : 0.f;
      sc = sig ? sigmoidf_(l) + b : l + b;
      vmax = fmaxf(vmax, sc);
    }
    raw[j] = l;
    v[j] = sc;
  }
  // the softmax-first rule reports probabilities: all-expert normaliser
  float zall = 1.f;
  if (a.mode == 1) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, off));
    zall = 0.f;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j)
      if (lane + 64 * j < E) zall += expf(v[j] - vmax);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) zall += __shfl_xor(zall, off);
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
      for (int j = 0; j < kPerLane; ++j)
        if (v[j] > bv) {  // ids ascend within a lane: ties keep the lower id
          bv = v[j];
          br = raw[j];
          bi = lane + 64 * j;
        }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const float orw = __shfl_xor(br, off);
        const int oi = __shfl_xor(bi, off);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          br = orw;
          bi = oi;
        }
      }
      sv[r] = bv;
      sraw[r] = br;
      si[r] = bi;
#pragma unroll
      for (int j = 0; j < kPerLane; ++j)
        if (lane + 64 * j == bi) v[j] = -INFINITY;
    }
  }
  if (lane != 0) return;

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
#pragma unroll
  for (int k = 0; k < kMaxK; ++k)
    if (k < K) {
      a.idx[t * K + k] = si[k];
      a.g[t * K + k] = gk[k] * a.routed_scale;
    }
  float rs[kMaxK + 1];  // scores in the ranked space
#pragma unroll
  for (int r = 0; r <= kMaxK; ++r)
    rs[r] = (a.mode == 1 && r < nsel) ? expf(sv[r] - vmax) / zall : sv[r];
  if (a.gap) {
    float gp = INFINITY;
#pragma unroll
    for (int r = 1; r <= kMaxK; ++r)
      if (r == K && K < E) gp = rs[r - 1] - rs[r];
    a.gap[t] = gp;
  }
  if (a.top) {
#pragma unroll
    for (int r = 0; r <= kMaxK; ++r)
      if (r <= K) a.top[t * (K + 1) + r] = r < nsel ? rs[r] : -INFINITY;
  }
}

}  // namespace

hipError_t launch_router(const RouterArgs &a, int act_bf16, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
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
  const int splits = router_splits(a.T, a.d);
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
  hipError_t e = launch_dense(g, EPI_STORE_F32, act_bf16, s);
  if (e != hipSuccess) return e;
  select_kernel<<<static_cast<unsigned>((a.T + 3) / 4), 256, 0, s>>>(a, parts, splits,
                                                                      g.split_stride);
  return hipGetLastError();
}

}  // namespace moe
