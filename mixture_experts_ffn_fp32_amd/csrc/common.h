// Device helpers shared by the HIP kernels of libmoe.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 is carried as its 16-bit pattern.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware:
// v_cvt_pk_bf16_f32, two values per instruction).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const void *p, int64_t i) {
    return static_cast<const float *>(p)[i];
  }
  static __device__ __forceinline__ void store(void *p, int64_t i, float v) {
    static_cast<float *>(p)[i] = v;
  }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const void *p, int64_t i) {
    return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
  }
  static __device__ __forceinline__ void store(void *p, int64_t i, float v) {
    static_cast<uint16_t *>(p)[i] = f32_to_bf16(v);
  }
};

// Unpack a 16-byte chunk into floats: 8 bf16 or 4 fp32 values.
template <typename T> struct Chunk;
template <> struct Chunk<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void unpack(const uint4 &c, float *v) {
    v[0] = __uint_as_float(c.x);
    v[1] = __uint_as_float(c.y);
    v[2] = __uint_as_float(c.z);
    v[3] = __uint_as_float(c.w);
  }
  static __device__ __forceinline__ uint4 pack(const float *v) {
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                      __float_as_uint(v[3]));
  }
};
template <> struct Chunk<bf16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void unpack(const uint4 &c, float *v) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ uint4 pack(const float *v) {
    return make_uint4(f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3]),
                      f32x2_to_bf16x2(v[4], v[5]), f32x2_to_bf16x2(v[6], v[7]));
  }
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Exclusive scan over a block of exactly 1024 threads; one value per thread.
// `tmp` is __shared__ scratch of at least 16 ints. Returns the exclusive
// prefix and writes the block total to *total.
__device__ __forceinline__ int block_exscan_1024(int v, int *tmp, int *total) {
  // inclusive scan inside each wavefront (shuffles), then of the 16
  // wavefront totals by wavefront 0; three barriers in all
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  if (w == 0) {
    int s = lane < 16 ? tmp[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int y = __shfl_up(s, off);
      if (lane >= off) s += y;
    }
    if (lane < 16) tmp[lane] = s;
  }
  __syncthreads();
  const int incl = x + (w ? tmp[w - 1] : 0);
  *total = tmp[15];
  __syncthreads();  // tmp may be rewritten as soon as this returns
  return incl - v;
}

}  // namespace moe
