// Router: fp32 logits, top-(K+1) selection and routing weights.
//
// APEX-1 Mathematical Reference - Part 3, section 13.2: r = x W_router + b,
// top-K of r, g = softmax over the K selected. "A working MoE layer in
// PyTorch": softmax over all experts in fp32, top-K, renormalise (the same
// weights in exact arithmetic). "StableLatentMoE and QuantileBalancer": fp32
// router, sigmoid scores, bias-corrected top-(K+1), last candidate dropped,
// weights are the uncorrected sigmoid scores.
//
// One workgroup takes 16 tokens. Its 256 threads each own one expert of the
// current 256-expert block and accumulate that expert's 16 fp32 logits from
// LDS-staged tiles of x and W_router (fp32 FMA, k ascending). The logits of
// the 16 tokens then sit in LDS, and each wavefront selects for one token at
// a time: every lane holds E/64 scores, and K+1 rounds of a butterfly
// (value, lower id) max-reduction over the 64 lanes pick the experts.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kTok = 16;    // tokens per workgroup
constexpr int kDk = 16;     // k per LDS stage
constexpr int kEb = 256;    // experts per pass (one per thread)
constexpr int kMaxK = 16;
constexpr int kMaxE = 1024;
constexpr int kPerLane = kMaxE / 64;

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }

template <typename T>
__global__ __launch_bounds__(256) void router_kernel(RouterArgs a) {
  __shared__ float xs[kTok][kDk];
  __shared__ float wsm[kEb][kDk + 1];
  __shared__ float logit[kTok][kMaxE];

  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTok;
  const int ntok = static_cast<int>(min<int64_t>(kTok, a.T - t0));

  for (int eb = 0; eb < a.E; eb += kEb) {
    float acc[kTok];
#pragma unroll
    for (int m = 0; m < kTok; ++m) acc[m] = 0.f;
    for (int k0 = 0; k0 < a.d; k0 += kDk) {
      for (int i = tid; i < kTok * kDk; i += 256) {
        const int m = i / kDk, k = i % kDk;
        float v = 0.f;
        if (m < ntok && k0 + k < a.d) v = Elem<T>::load(a.x, (t0 + m) * a.d + k0 + k);
        xs[m][k] = v;
      }
      for (int i = tid; i < kEb * kDk; i += 256) {
        const int r = i / kDk, k = i % kDk;
        float v = 0.f;
        if (eb + r < a.E && k0 + k < a.d) v = a.w[static_cast<int64_t>(eb + r) * a.d + k0 + k];
        wsm[r][k] = v;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kDk; ++k) {
        const float wv = wsm[tid][k];
#pragma unroll
        for (int m = 0; m < kTok; ++m) acc[m] = fmaf(xs[m][k], wv, acc[m]);
      }
      __syncthreads();
    }
    if (eb + tid < a.E) {
#pragma unroll
      for (int m = 0; m < kTok; ++m) logit[m][eb + tid] = acc[m];
    }
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63;
  const int E = a.E, K = a.K;
  const int nsel = K + 1 <= E ? K + 1 : E;
  const bool sig = a.mode == 2;
  for (int m = wave; m < ntok; m += 4) {
    const int64_t t = t0 + m;
    float v[kPerLane];
    float vmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      const int e = lane + 64 * j;
      float sc = -INFINITY;
      if (e < E) {
        const float l = logit[m][e];
        const float b = a.bias ? a.bias[e] : 0.f;
        sc = sig ? sigmoidf_(l) + b : l + b;
        vmax = fmaxf(vmax, sc);
      }
      v[j] = sc;
    }
    // softmax-first rule reports probabilities: need the all-expert sum
    float zall = 0.f;
    if (a.mode == 1) {
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, off));
#pragma unroll
      for (int j = 0; j < kPerLane; ++j)
        if (lane + 64 * j < E) zall += expf(v[j] - vmax);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) zall += __shfl_xor(zall, off);
    }

    float sv[kMaxK + 1];
    int si[kMaxK + 1];
#pragma unroll
    for (int r = 0; r <= kMaxK; ++r) {
      sv[r] = -INFINITY;
      si[r] = 0;
      if (r < nsel) {
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int j = 0; j < kPerLane; ++j)
          if (v[j] > bv) {  // ascending id within the lane: ties keep the lower id
            bv = v[j];
            bi = lane + 64 * j;
          }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
          const float ov = __shfl_xor(bv, off);
          const int oi = __shfl_xor(bi, off);
          if (ov > bv || (ov == bv && oi < bi)) {
            bv = ov;
            bi = oi;
          }
        }
        sv[r] = bv;
        si[r] = bi;
#pragma unroll
        for (int j = 0; j < kPerLane; ++j)
          if (lane + 64 * j == bi) v[j] = -INFINITY;
      }
    }

    if (lane == 0) {
      float gk[kMaxK];
      float z = 0.f;
      if (sig) {
#pragma unroll
        for (int k = 0; k < kMaxK; ++k)
          if (k < K) {
            gk[k] = sigmoidf_(logit[m][si[k]]);
            z += gk[k];
          }
        if (a.renormalize) {
#pragma unroll
          for (int k = 0; k < kMaxK; ++k)
            if (k < K) gk[k] = gk[k] / z;
        }
      } else {
        const float top = sv[0];
#pragma unroll
        for (int k = 0; k < kMaxK; ++k)
          if (k < K) {
            gk[k] = expf(sv[k] - top);
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
      // scores in the ranked space (probabilities for the softmax-first rule)
      float rs[kMaxK + 1];
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
  }
}

}  // namespace

hipError_t launch_router(const RouterArgs &a, int act_bf16, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((a.T + kTok - 1) / kTok));
  if (act_bf16)
    router_kernel<bf16_t><<<grid, 256, 0, s>>>(a);
  else
    router_kernel<float><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
