// Grouped / dense GEMM on CDNA4 matrix cores with fused MoE epilogues.
//
// C = A B^T: A [M, K] activations (rows optionally gathered through an index,
// which fuses the dispatch gather into the operand load), B [N, K] weights
// stored "out x in". Grouped mode ("StableLatentMoE and QuantileBalancer",
// "The actual grouped GEMM"): a device-built table lists m-tiles as
// {expert, row_begin, row_end} over the expert-sorted rows, so experts with
// no rows get no tile and a skewed expert spreads over many tiles, with no
// host round trip. Dense mode: one group of M rows.
//
// Epilogues:
//   SWIGLU  - B holds gate rows and up rows for the same output columns;
//             out = SiLU(x W_gate^T) * (x W_up^T)  (APEX-1 Math. Reference
//             Part 3, 12.2), rounded to the activation type;
//   SCALE   - out = row_scale[m] * acc (the routing weight of the row);
//   STORE   - out = acc (optionally over two K segments: out = A1 B1^T +
//             A2 B2^T, used for shared-down + latent-up in one pass);
//   STORE_F32 - out = acc kept in fp32 (router logits);
//   COMBINE - out[t] = acc + sum_k y[inv[t*K + k]] in fixed k order: the
//             shared expert's down projection and the atomic-free combine
//             of the routed rows (Math. Reference 13.2) in one pass.
//
// Kernel shape: 256 threads (4 wavefronts). Per stage the workgroup stages a
// BM x 128-byte slab of A and a BN x 128-byte slab of B in LDS with 16-byte
// global loads (8 lanes per row), double-buffered so the next stage's loads
// are in flight during the current stage's MFMAs. Rows of a slab are XOR
// swizzled in 16-byte units so the 16-byte fragment reads of 8 consecutive
// rows fall in distinct LDS bank groups. Each wavefront owns a
// (BM/WM) x (BN/WN) block of 16x16 accumulators: bf16 uses
// v_mfma_f32_16x16x32_bf16 (one 16-byte fragment per lane per MFMA), fp32
// uses four v_mfma_f32_16x16x4_f32 per fragment.
//
// Block order: blocks are dealt round-robin to the 8 XCDs, so block b is
// mapped to tile index (b % 8) * per_xcd + b / 8: each XCD works through a
// contiguous stretch of the tile list, and consecutive tiles are grouped 4
// m-tiles at a time across the n-tiles so the A and B panels they share are
// reused from that XCD's L2.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__device__ __forceinline__ int swz(int r, int kc) { return r * 8 + (kc ^ (r & 7)); }

template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
  static __device__ __forceinline__ void run(const uint4 &a, const uint4 &b, f32x4 &c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  static __device__ __forceinline__ void run(const uint4 &a, const uint4 &b, f32x4 &c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
};

// SiLU with the hardware reciprocal (1 ulp) in place of an IEEE division:
// the product is rounded to bf16 or kept in fp32 within the layer's tolerance
__device__ __forceinline__ float silu_f(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

template <typename T, int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(GemmArgs p) {
  constexpr int THREADS = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int ES = static_cast<int>(sizeof(T));
  constexpr int EPC = 16 / ES;  // elements per 16-byte chunk
  constexpr int BK = 8 * EPC;   // k per stage (128 bytes per row)
  constexpr bool GLU = EPI == EPI_SWIGLU;
  constexpr int NOUT = GLU ? BN / 2 : BN;
  constexpr int A_CH = BM * 8, B_CH = BN * 8;
  constexpr int A_LD = (A_CH + THREADS - 1) / THREADS;
  constexpr int B_LD = (B_CH + THREADS - 1) / THREADS;
  constexpr int ROWS_PER_PASS = THREADS / 8;
  static_assert(!GLU || FN % 2 == 0, "SwiGLU needs paired gate/up fragments");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "fragments are 16x16");

  __shared__ uint4 lds[2][(BM + BN) * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---------------------------------------------------------------- tile
  const int n_tn = (p.N + NOUT - 1) / NOUT;
  const int64_t n_m = p.tiles ? static_cast<int64_t>(*p.n_tiles) : p.max_mtiles;
  const int ksplit = p.k_split > 1 ? p.k_split : 1;
  const int64_t total = n_m * n_tn * ksplit;
  const int64_t per = (total + 7) / 8;
  const int64_t local = blockIdx.x >> 3;
  if (local >= per) return;
  const int64_t pid = static_cast<int64_t>(blockIdx.x & 7) * per + local;
  if (pid >= total) return;
  const int64_t tiles2d = n_m * n_tn;
  const int split = static_cast<int>(pid / tiles2d);
  const int64_t tpid = pid - split * tiles2d;
  constexpr int GM = 4;
  const int64_t grp = tpid / (GM * n_tn);
  const int64_t first_m = grp * GM;
  const int gsz = static_cast<int>(min<int64_t>(n_m - first_m, GM));
  const int64_t in_g = tpid - grp * GM * n_tn;
  const int64_t mt = first_m + in_g % gsz;
  const int nt = static_cast<int>(in_g / gsz);
  int64_t expert = 0, m_begin, m_end;
  if (p.tiles) {
    expert = p.tiles[kTileInts * mt];
    m_begin = p.tiles[kTileInts * mt + 1];
    m_end = p.tiles[kTileInts * mt + 2];
  } else {
    m_begin = mt * BM;
    m_end = min<int64_t>(m_begin + BM, p.M);
  }
  const int n_begin = nt * NOUT;
  // K-grouped: this expert's reduction columns and output block
  int64_t kbeg = 0;
  int kseg = p.K;
  if (p.k_offsets) {
    kbeg = p.k_offsets[expert];
    kseg = static_cast<int>(p.k_offsets[expert + 1] - kbeg);
  }
  const int64_t obase = p.k_offsets ? expert * p.out_stride : 0;

  // ---------------------------------------------------------------- loaders
  const int kc_ld = tid & 7;
  const char *arow[A_LD];
  const char *brow[B_LD];
  auto setup = [&](int seg) {
    const char *abase = static_cast<const char *>(seg ? p.a2 : p.a);
    const int64_t lda = seg ? p.lda2 : p.lda;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int r = (tid >> 3) + i * ROWS_PER_PASS;
      const int64_t m = m_begin + r;
      arow[i] = nullptr;
      if (r < BM && m < m_end) {
        const int64_t src = (!seg && p.a_rows) ? static_cast<int64_t>(p.a_rows[m]) : m;
        arow[i] = abase + (src * lda + (seg ? 0 : kbeg)) * ES;
      }
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int r = (tid >> 3) + i * ROWS_PER_PASS;
      brow[i] = nullptr;
      if (r < BN) {
        const char *bbase;
        int n;
        int64_t ldb, off = 0;
        if (seg) {
          bbase = static_cast<const char *>(p.b2);
          n = n_begin + r;
          ldb = p.ldb2;
        } else {
          const bool up = GLU && r >= BN / 2;
          bbase = static_cast<const char *>(up ? p.b1 : p.b0);
          n = n_begin + (up ? r - BN / 2 : r);
          ldb = p.ldb;
          off = expert * p.b_stride + kbeg;
        }
        if (n < p.N) brow[i] = bbase + (off + static_cast<int64_t>(n) * ldb) * ES;
      }
    }
  };

  const int steps1 = (kseg + BK - 1) / BK;
  const int steps = steps1 + (p.a2 ? (p.K2 + BK - 1) / BK : 0);
  // this split's stages (single-segment GEMMs only are split)
  const int per_split = (steps + ksplit - 1) / ksplit;
  const int st_begin = min(steps, split * per_split);
  const int st_end = min(steps, st_begin + per_split);
  uint4 ra[A_LD], rb[B_LD];
  auto load = [&](int st) {
    const bool s2 = st >= steps1;
    const int k = (s2 ? st - steps1 : st) * BK + kc_ld * EPC;
    const bool kin = k < (s2 ? p.K2 : kseg);
    const int64_t kb = static_cast<int64_t>(k) * ES;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      ra[i] = make_uint4(0, 0, 0, 0);
      if (kin && arow[i]) ra[i] = *reinterpret_cast<const uint4 *>(arow[i] + kb);
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      rb[i] = make_uint4(0, 0, 0, 0);
      if (kin && brow[i]) rb[i] = *reinterpret_cast<const uint4 *>(brow[i] + kb);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int r = (tid >> 3) + i * ROWS_PER_PASS;
      if (r < BM) lds[buf][swz(r, kc_ld)] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int r = (tid >> 3) + i * ROWS_PER_PASS;
      if (r < BN) lds[buf][BM * 8 + swz(r, kc_ld)] = rb[i];
    }
  };

  // B row (within the slab) of this wave's fragment fn
  auto bfrag_row = [&](int fn) {
    if (GLU) {
      const int half = FN / 2;
      return fn < half ? wn * (WTN / 2) + fn * 16 : BN / 2 + wn * (WTN / 2) + (fn - half) * 16;
    }
    return wn * WTN + fn * 16;
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  setup(0);
  if (st_begin < st_end) {
    load(st_begin);
    store(0);
    __syncthreads();
  }
  for (int st = st_begin; st < st_end; ++st) {
    const int cur = (st - st_begin) & 1;
    const bool more = st + 1 < st_end;
    if (more) {
      if (st + 1 == steps1) setup(1);
      load(st + 1);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kc = 4 * s + (lane >> 4);
      uint4 af[FM], bfr[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        af[fm] = lds[cur][swz(wm * WTM + fm * 16 + (lane & 15), kc)];
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        bfr[fn] = lds[cur][BM * 8 + swz(bfrag_row(fn) + (lane & 15), kc)];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) Mfma<T>::run(af[fm], bfr[fn], acc[fm][fn]);
    }
    if (more) store(cur ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  constexpr int FO = GLU ? FN / 2 : FN;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m_begin + wm * WTM + fm * 16 + 4 * (lane >> 4) + r;
      if (m >= m_end) continue;
      float rsc = 1.0f;
      if (EPI == EPI_SCALE && p.row_scale) rsc = p.row_scale[m];
#pragma unroll
      for (int fo = 0; fo < FO; ++fo) {
        const int col = n_begin + (GLU ? wn * (WTN / 2) : wn * WTN) + fo * 16 + (lane & 15);
        if (col >= p.N) continue;
        float v;
        if (GLU) {
          v = silu_f(acc[fm][fo][r]) * acc[fm][fo + FO][r];
        } else if (EPI == EPI_SCALE) {
          v = acc[fm][fo][r] * rsc;
        } else if (EPI == EPI_COMBINE) {
          v = acc[fm][fo][r];
          float rs = 0.f;
          for (int k = 0; k < p.topk; ++k) {
            const int q = p.inv[m * p.topk + k];
            if (q >= 0) rs += Elem<T>::load(p.y, static_cast<int64_t>(q) * p.ldy + col);
          }
          v += rs;
        } else {
          v = acc[fm][fo][r];
        }
        if (EPI == EPI_STORE_F32 || (EPI == EPI_SCALE && p.out_f32))
          static_cast<float *>(p.out)[obase + split * p.split_stride + m * p.ldo + col] = v;
        else
          Elem<T>::store(p.out, m * p.ldo + col, v);
      }
    }
  }
}

struct CfgSmallM {  // few rows per expert (decode): stream B
  static constexpr int BM = 16, BN = 256, WM = 1, WN = 4;
};
struct CfgLarge {
  static constexpr int BM = 128, BN = 128, WM = 2, WN = 2;
};
struct CfgTallN64 {  // few output columns: half-width tiles
  static constexpr int BM = 128, BN = 64, WM = 2, WN = 2;
};
struct CfgMid {  // small problems: more, smaller tiles
  static constexpr int BM = 64, BN = 64, WM = 2, WN = 2;
};
struct CfgSmallN64 {  // few rows (decode-sized dense GEMMs): narrow tiles, many workgroups
  static constexpr int BM = 16, BN = 64, WM = 1, WN = 2;
};
struct CfgWide {
  static constexpr int BM = 128, BN = 256, WM = 2, WN = 2;
};
struct CfgTall {
  static constexpr int BM = 256, BN = 128, WM = 2, WN = 2;
};
struct CfgHuge {
  static constexpr int BM = 256, BN = 256, WM = 2, WN = 2;
};

template <typename T, typename C, int EPI>
hipError_t run(const GemmArgs &a, hipStream_t s) {
  if (a.k_split > 1 && (EPI != EPI_STORE_F32 || a.a2)) return hipErrorInvalidValue;
  constexpr int NOUT = EPI == EPI_SWIGLU ? C::BN / 2 : C::BN;
  const int64_t n_tn = (a.N + NOUT - 1) / NOUT;
  const int64_t max_m = a.tiles ? a.max_mtiles : (a.M + C::BM - 1) / C::BM;
  const int64_t total = max_m * n_tn * (a.k_split > 1 ? a.k_split : 1);
  if (total == 0) return hipSuccess;
  GemmArgs b = a;
  b.max_mtiles = max_m;
  const int64_t blocks = 8 * ((total + 7) / 8);
  gemm_kernel<T, C::BM, C::BN, C::WM, C::WN, EPI>
      <<<static_cast<unsigned>(blocks), 64 * C::WM * C::WN, 0, s>>>(b);
  return hipGetLastError();
}

template <typename T, typename C>
hipError_t dispatch_epi(const GemmArgs &a, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_SWIGLU: return run<T, C, EPI_SWIGLU>(a, s);
    case EPI_SCALE: return run<T, C, EPI_SCALE>(a, s);
    case EPI_STORE: return run<T, C, EPI_STORE>(a, s);
    case EPI_COMBINE: return run<T, C, EPI_COMBINE>(a, s);
    case EPI_STORE_F32: return run<T, C, EPI_STORE_F32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

template <typename C>
int64_t tiles_of(int64_t rows, int64_t n_out, int glu) {
  const int64_t nout = glu ? C::BN / 2 : C::BN;
  return ((rows + C::BM - 1) / C::BM) * ((n_out + nout - 1) / nout);
}

int64_t tile_count(int cfg, int64_t rows, int64_t n_out, int glu) {
  switch (cfg) {
    case TILE_SMALL_M: return tiles_of<CfgSmallM>(rows, n_out, glu);
    case TILE_MID: return tiles_of<CfgMid>(rows, n_out, glu);
    case TILE_TALL_N64: return tiles_of<CfgTallN64>(rows, n_out, glu);
    case TILE_SMALL_N64: return tiles_of<CfgSmallN64>(rows, n_out, glu);
    default: return tiles_of<CfgLarge>(rows, n_out, glu);
  }
}

int tile_bm(int cfg) {
  switch (cfg) {
    case TILE_MID: return CfgMid::BM;
    case TILE_TALL_N64: return CfgTallN64::BM;
    case TILE_SMALL_N64: return CfgSmallN64::BM;
    case TILE_SMALL_M: return CfgSmallM::BM;
    case TILE_LARGE: return CfgLarge::BM;
    case TILE_WIDE: return CfgWide::BM;
    case TILE_TALL: return CfgTall::BM;
    case TILE_HUGE: return CfgHuge::BM;
  }
  return CfgLarge::BM;
}

int tile_bn(int cfg) {
  switch (cfg) {
    case TILE_MID: return CfgMid::BN;
    case TILE_TALL_N64: return CfgTallN64::BN;
    case TILE_SMALL_N64: return CfgSmallN64::BN;
    case TILE_SMALL_M: return CfgSmallM::BN;
    case TILE_LARGE: return CfgLarge::BN;
    case TILE_WIDE: return CfgWide::BN;
    case TILE_TALL: return CfgTall::BN;
    case TILE_HUGE: return CfgHuge::BN;
  }
  return CfgLarge::BN;
}

hipError_t launch_gemm(const GemmArgs &a, int epi, int cfg, int act_bf16, hipStream_t s) {
  if (!act_bf16)  // fp32 runs the two base shapes only
    return cfg == TILE_SMALL_M ? dispatch_epi<float, CfgSmallM>(a, epi, s)
                               : dispatch_epi<float, CfgLarge>(a, epi, s);
  switch (cfg) {
    case TILE_SMALL_M: return dispatch_epi<bf16_t, CfgSmallM>(a, epi, s);
    case TILE_MID: return dispatch_epi<bf16_t, CfgMid>(a, epi, s);
    case TILE_TALL_N64: return dispatch_epi<bf16_t, CfgTallN64>(a, epi, s);
    case TILE_SMALL_N64: return dispatch_epi<bf16_t, CfgSmallN64>(a, epi, s);
    case TILE_WIDE: return dispatch_epi<bf16_t, CfgWide>(a, epi, s);
    case TILE_TALL: return dispatch_epi<bf16_t, CfgTall>(a, epi, s);
    case TILE_HUGE: return dispatch_epi<bf16_t, CfgHuge>(a, epi, s);
    default: return dispatch_epi<bf16_t, CfgLarge>(a, epi, s);
  }
}

}  // namespace moe
