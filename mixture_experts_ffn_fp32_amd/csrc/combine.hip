// Atomic-free combine of the routed rows through the inverse permutation.
//
// APEX-1 Mathematical Reference - Part 3, 13.2: the routed part of token t is
// sum_k g_k Expert_{e_k}(x_t). The grouped GEMM has already multiplied each
// sorted row by its g, so token t's routed part is the sum of its K rows at
// sorted positions inv[t*K + k] ("StableLatentMoE and QuantileBalancer": the
// permutation is undone when contributions return to their token rows). Each
// output row is produced by one workgroup, summing in fixed k order in fp32:
// no atomics, and the result does not depend on scheduling.
//
// The latent variant ("StableLatentMoE", "Return to model width") then
// applies RMSNorm in the latent width: R / sqrt(mean(R^2) + eps) * gamma.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// out[t] = sum_k y[inv[t*K+k]] (+ add[t], fp32): one wavefront per token and
// span of 64 * cstep chunks (blockIdx.y), 16-byte chunks, the K rows summed
// in k order in fp32, then add.
template <typename T>
__global__ __launch_bounds__(256) void combine_sum_kernel(const uint4 *__restrict__ y,
                                                          const int32_t *__restrict__ inv, int K,
                                                          int chunks, int64_t n_tok,
                                                          const float *__restrict__ add,
                                                          uint4 *__restrict__ out, int cspan) {
  constexpr int N = Chunk<T>::N;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= n_tok) return;
  const int c_end = min(chunks, static_cast<int>(blockIdx.y + 1) * cspan);
  constexpr int kMaxSlots = 16;
  int q[kMaxSlots];  // the token's sorted rows, read once
#pragma unroll
  for (int k = 0; k < kMaxSlots; ++k) q[k] = k < K ? inv[t * K + k] : -1;
  for (int c = blockIdx.y * cspan + (threadIdx.x & 63); c < c_end; c += 64) {
    uint4 raw[kMaxSlots];  // all K rows requested before they are added
#pragma unroll
    for (int k = 0; k < kMaxSlots; ++k)
      raw[k] = q[k] >= 0 ? y[static_cast<int64_t>(q[k]) * chunks + c] : make_uint4(0u, 0u, 0u, 0u);
    float acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxSlots; ++k) {
      if (q[k] < 0) continue;
      float v[N];
      Chunk<T>::unpack(raw[k], v);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += v[i];
    }
    if (add) {
      const float4 *a4 = reinterpret_cast<const float4 *>(add + (t * chunks + c) * N);
#pragma unroll
      for (int i = 0; i < N / 4; ++i) {
        const float4 v = a4[i];
        acc[4 * i] += v.x;
        acc[4 * i + 1] += v.y;
        acc[4 * i + 2] += v.z;
        acc[4 * i + 3] += v.w;
      }
    }
    out[t * chunks + c] = Chunk<T>::pack(acc);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void combine_latent_kernel(const uint4 *__restrict__ y,
                                                             const int32_t *__restrict__ inv,
                                                             int K, int chunks, int L,
                                                             int has_rmsnorm, float eps,
                                                             const float *__restrict__ gamma,
                                                             uint4 *__restrict__ r) {
  // one workgroup per token, a thread per 16-byte chunk of the row (the
  // workgroup is as wide as the row, in whole wavefronts, up to 256
  // threads; wider rows loop and keep their sums in LDS). Each chunk's K
  // rows are all requested before they are added, in slot order.
  constexpr int N = Chunk<T>::N;
  constexpr int kMaxSlots = 16;
  extern __shared__ float row[];  // [L], for rows wider than the workgroup
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const int nthr = blockDim.x;
  const bool one = chunks <= nthr;  // one chunk per thread: sums stay in registers
  int q[kMaxSlots];
#pragma unroll
  for (int k = 0; k < kMaxSlots; ++k) q[k] = k < K ? inv[t * K + k] : -1;
  float keep[N];
  float ss = 0.f;
  for (int c = threadIdx.x; c < chunks; c += nthr) {
    uint4 raw[kMaxSlots];
#pragma unroll
    for (int k = 0; k < kMaxSlots; ++k)
      raw[k] = q[k] >= 0 ? y[static_cast<int64_t>(q[k]) * chunks + c] : make_uint4(0u, 0u, 0u, 0u);
    float acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxSlots; ++k) {
      if (q[k] < 0) continue;
      float v[N];
      Chunk<T>::unpack(raw[k], v);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += v[i];
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      keep[i] = acc[i];
      if (!one) row[c * N + i] = acc[i];
      ss += acc[i] * acc[i];
    }
  }
  float scale = 1.0f;
  if (has_rmsnorm) {  // per wavefront, then the wavefronts in order
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int w = 0; w < nthr / 64; ++w) tot += red[w];
    scale = 1.0f / sqrtf(tot / static_cast<float>(L) + eps);
  }
  if (!one) __syncthreads();
  for (int c = threadIdx.x; c < chunks; c += nthr) {
    float v[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int l = c * N + i;
      const float x = one ? keep[i] : row[l];
      v[i] = has_rmsnorm ? x * scale * (gamma ? gamma[l] : 1.0f) : x;
    }
    r[t * chunks + c] = Chunk<T>::pack(v);
  }
}

}  // namespace

hipError_t launch_combine_sum(const void *y, const int32_t *inv, int64_t T, int K, int width,
                              void *out, int act_bf16, hipStream_t s, const float *add) {
  if (T == 0) return hipSuccess;
  if (K > 16) return hipErrorInvalidValue;
  const int chunks = width / (act_bf16 ? 8 : 4);
  // few tokens: split each row over column spans (multiples of 64 chunks) so
  // that the launch has about 1024 wavefronts
  const int64_t waves_per_tok = (1024 + T - 1) / T;
  int64_t span = (chunks + waves_per_tok - 1) / waves_per_tok;
  span = (span + 63) / 64 * 64;
  const int cspan = static_cast<int>(span < chunks ? span : chunks);
  const dim3 grid(static_cast<unsigned>((T + 3) / 4), static_cast<unsigned>((chunks + cspan - 1) / cspan));
  if (act_bf16)
    combine_sum_kernel<bf16_t><<<grid, 256, 0, s>>>(static_cast<const uint4 *>(y), inv, K, chunks,
                                                    T, add, static_cast<uint4 *>(out), cspan);
  else
    combine_sum_kernel<float><<<grid, 256, 0, s>>>(static_cast<const uint4 *>(y), inv, K, chunks,
                                                   T, add, static_cast<uint4 *>(out), cspan);
  return hipGetLastError();
}

hipError_t launch_combine_latent(const void *y, const int32_t *inv, int64_t T, int K, int L,
                                 int has_rmsnorm, float eps, const float *gamma, void *r,
                                 int act_bf16, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (K > 16) return hipErrorInvalidValue;
  const int chunks = L / (act_bf16 ? 8 : 4);
  const int nthr = chunks >= 256 ? 256 : (chunks + 63) / 64 * 64;
  const size_t shm = chunks > nthr ? static_cast<size_t>(L) * sizeof(float) : 0;
  if (act_bf16)
    combine_latent_kernel<bf16_t><<<static_cast<unsigned>(T), nthr, shm, s>>>(
        static_cast<const uint4 *>(y), inv, K, chunks, L, has_rmsnorm, eps, gamma,
        static_cast<uint4 *>(r));
  else
    combine_latent_kernel<float><<<static_cast<unsigned>(T), nthr, shm, s>>>(
        static_cast<const uint4 *>(y), inv, K, chunks, L, has_rmsnorm, eps, gamma,
        static_cast<uint4 *>(r));
  return hipGetLastError();
}

}  // namespace moe
