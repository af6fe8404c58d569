// Peak-rate microbenchmarks of the part, for the measurement side of the
// library (not a step of the layer): back-to-back independent bf16 MFMAs of
// either shape, conflict-free 16-byte LDS reads, and the two mixed in the
// ratio a GEMM's main loop issues them (each MFMA group's operands read from
// LDS half an iteration earlier, as the pipelined GEMM does). Every
// workgroup reads the shader clock (s_memtime) and the constant 100 MHz
// clock (s_memrealtime) around its loop, so the host can derive the running
// shader clock and the per-CU issue rates.
//
// One workgroup per CU: each holds 96 KB of LDS, so no second one fits.
// 256 threads put one wavefront on each SIMD, 512 two.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPeakLds16 = 96 * 1024 / 16;  // 16-byte units of LDS per workgroup
constexpr int kReadMask = 4096 - 1;         // reads cycle through the first 64 KB

// 16-byte unit read by `lane` for read number q of a wavefront under the
// fragment pattern PAT (LDS rows of 128 bytes, 8 units each, as a GEMM
// stage buffer holds 64 bf16 of k per row): 0 contiguous (lane i reads unit
// i); 1 / 2 the 16x16x32 operand (16 rows, lanes 16 apart take the next
// 8-k unit) with units XOR-swizzled by row & 7 / by (row >> 1) & 7; 3 / 4
// the 32x32x16 operand (32 rows, lanes 32 apart take the next unit), same
// two swizzles.
template <int PAT>
__device__ __forceinline__ int frag_unit(int wave, int lane, int q) {
  if (PAT == 0) return (wave * 512 + q * 64 + lane) & kReadMask;
  const int rows = PAT <= 2 ? 16 : 32;
  const int r = lane % rows, u = lane / rows;
  // successive reads step 24 / 40 rows (not a power of two: the addresses
  // repeat only after 64 reads, so no read is loop-invariant)
  const int row = (wave * 64 + q * (rows + 8) + r) & 511;
  const int kc = ((q & 1) * 4 + u) & 7;
  const int sw = (PAT == 1 || PAT == 3) ? (row & 7) : ((row >> 1) & 7);
  return row * 8 + (kc ^ sw);
}

// KIND 0: v_mfma_f32_16x16x32_bf16, 8 per half-iteration; KIND 1:
// v_mfma_f32_32x32x16_bf16, 4 per half-iteration (131072 flops either way);
// KIND 2: LDS reads only. RD: 16-byte LDS reads per half-iteration. PAT:
// the read pattern (frag_unit).
template <int KIND, int RD, int PAT = 0>
__global__ __launch_bounds__(512) void peak_kernel(int iters, int64_t *clk, uint32_t *sink) {
  __shared__ __attribute__((aligned(1024))) uint4 lds[kPeakLds16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kPeakLds16; i += blockDim.x)
    lds[i] = make_uint4(0x3F803F80u + (i & 7), 0x3F003F80u, 0x3F803F00u, 0x3E803F80u);
  __syncthreads();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();

  constexpr int NB = RD > 0 ? RD : 1;
  constexpr int NM = KIND == 0 ? 8 : 4;
  const __bf16 one = static_cast<__bf16>(1.0f + lane * 0.0078125f);
  bf16x8 buf[2][NB];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int r = 0; r < NB; ++r) buf[h][r] = bf16x8{one, one, one, one, one, one, one, one};
  f32x4 acc4[8];
  f32x16 acc16[4];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc4[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc16[j][e] = 0.f;
  uint4 x = make_uint4(0, 0, 0, 0);

  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // this half's reads (operands of the next half's MFMAs)
#pragma unroll
      for (int r = 0; r < RD; ++r) {
        const uint4 v = lds[frag_unit<PAT>(wave, lane, (2 * it + h) * RD + r)];
        if (KIND == 2) {
          x.x ^= v.x;
          x.y ^= v.y;
          x.z ^= v.z;
          x.w ^= v.w;
        } else {
          buf[h ^ 1][r] = __builtin_bit_cast(bf16x8, v);
        }
      }
      if constexpr (KIND == 0) {
#pragma unroll
        for (int j = 0; j < NM; ++j)
          acc4[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(buf[h][j % NB], buf[h][(j + 1) % NB],
                                                            acc4[j], 0, 0, 0);
      } else if constexpr (KIND == 1) {
#pragma unroll
        for (int j = 0; j < NM; ++j)
          acc16[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(buf[h][j % NB], buf[h][(j + 1) % NB],
                                                             acc16[j], 0, 0, 0);
      }
    }
  }
  __syncthreads();
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (RD == 0) x = lds[tid & kReadMask];  // keeps the 96 KB allocated: one workgroup per CU
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc4[j][0] + acc4[j][3];
#pragma unroll
  for (int j = 0; j < 4; ++j) s += acc16[j][0] + acc16[j][15];
  sink[static_cast<int64_t>(blockIdx.x) * blockDim.x + tid] =
      __float_as_uint(s) ^ x.x ^ x.y ^ x.z ^ x.w;
  if (tid == 0) {
    clk[2 * blockIdx.x] = static_cast<int64_t>(c1 - c0);
    clk[2 * blockIdx.x + 1] = static_cast<int64_t>(r1 - r0);
  }
}

template <int KIND, int RD, int PAT = 0>
hipError_t run_peak(int threads, int groups, int iters, int64_t *clk, uint32_t *sink,
                    hipStream_t s) {
  peak_kernel<KIND, RD, PAT><<<groups, threads, 0, s>>>(iters, clk, sink);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_peak(int mode, int threads, int groups, int iters, int64_t *clk,
                       uint32_t *sink, hipStream_t s) {
  switch (mode) {
    case 0: return run_peak<0, 0>(threads, groups, iters, clk, sink, s);
    case 1: return run_peak<1, 0>(threads, groups, iters, clk, sink, s);
    case 2: return run_peak<2, 8>(threads, groups, iters, clk, sink, s);
    case 3: return run_peak<0, 3>(threads, groups, iters, clk, sink, s);
    case 4: return run_peak<1, 3>(threads, groups, iters, clk, sink, s);
    case 5: return run_peak<0, 2>(threads, groups, iters, clk, sink, s);
    case 6: return run_peak<1, 2>(threads, groups, iters, clk, sink, s);
    case 7: return run_peak<2, 8, 1>(threads, groups, iters, clk, sink, s);
    case 8: return run_peak<2, 8, 2>(threads, groups, iters, clk, sink, s);
    case 9: return run_peak<2, 8, 3>(threads, groups, iters, clk, sink, s);
    case 10: return run_peak<2, 8, 4>(threads, groups, iters, clk, sink, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
