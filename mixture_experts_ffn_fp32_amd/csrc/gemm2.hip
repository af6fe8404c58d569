// Pipelined bf16 GEMM for large tiles (gfx950): C = A B^T, same contract and
// epilogues as gemm.hip (grouped expert tiles from a device table or dense;
// row-gathered A; SwiGLU, row-scale, store, fp32 store, combine epilogues;
// optional second K segment).
//
// Work split. A workgroup of WGM x WGN wavefronts owns a BM x BN tile; each
// wavefront holds a (BM/WGM) x (BN/WGN) block of 16x16 fp32 accumulators fed
// by v_mfma_f32_16x16x32_bf16. The 256x256 tile runs 8 wavefronts (two per
// SIMD): one wavefront alone cannot issue MFMAs back to back at the full rate
// nor keep the LDS busy, and the second hides the first's waits.
//
// Loads. K advances 64 elements (128 bytes per row) per stage. Operand rows
// go straight from global memory to LDS with 16-byte buffer loads: lane i of
// a load lands at byte 16 i of a 1 KB block of 8 rows, and the eight 16-byte
// chunks of a row are XOR-swizzled by row & 7 (so the fragment reads of 8
// consecutive rows hit distinct banks); each lane therefore fetches the
// logical chunk its slot holds. A has NA stage buffers and B NA + 1, so the
// streamed weights are requested NA stages ahead and the activations NA - 1
// (NA = 2 for the 256x256 tiles, which fill the LDS; up to 4 for smaller
// tiles, whose short K loops are bound by load latency rather than MFMAs).
// Offsets are 32-bit against per-operand buffer resources (extents below
// 4 GiB are a launch precondition); B rows past N lie past the resource's
// extent and read as zeros; A rows past the tile's end repeat its first row
// (their results are never stored).
//
// Main loop, per stage s (A buffer s % NA, B buffer s % (NA + 1)), fragments in two
// register sets (set 0: k-step 0, set 1: k-step 1):
//   M0: MFMAs of set 0, interleaved row by row with the LDS reads of set 1;
//   wait until stage s + 1 has landed (later stages may still be in flight),
//       lgkmcnt 0, barrier: stage s + 1 is visible and stage s's buffers
//       are free;
//   M1: MFMAs of set 1, interleaved with the loads of A(s + NA) and B(s + NA + 1)
//       into the freed buffers and the reads of stage s + 1's k-step 0.
// Each MFMA group's operands were requested half a stage earlier. Loads past
// the last stage repeat it (their buffers are never read), so every stage
// issues the same number of loads and the wait counts are constants.
// sched_barrier keeps the interleaving in program order.
//
// Epilogue. Each wavefront stages its accumulators through LDS 16 rows at a
// time and writes the output with 16-byte stores along rows; the combine
// epilogue adds the token's K routed rows with 16-byte loads. The plain fp32
// store writes straight from the accumulators (64-byte row pieces).
//
// K-major B (template flag BKM, fp32-store epilogue only): B given as
// [K, N] row-major, as the backward's products read W_down, W_gate and W_up
// in place. A stage buffer then holds 64 k-rows of the tile's columns and
// fragments come from transposing LDS reads (ds_read_b64_tr_b16).
//
// K must be a multiple of 32 (the first of two K segments, of 64); the host
// uses gemm.hip otherwise.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// dense launches: m-tiles per tile group (the group runs over all n-tiles)
constexpr int kGroupM = 4;

// bytes of one operand row per stage (64 bf16)
constexpr int kRowBytes = 128;

// s_waitcnt with vmcnt = N (< 64), lgkmcnt = 0, expcnt untouched.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// 16-byte direct-to-LDS load: lane i's data lands at lds + 16 i (lds is
// wave-uniform). (Device-pass only: the host pass does not know the builtin.)
//
// UNTRACKED: the same load issued from inline asm, which the compiler does
// not see as an LDS write. It cannot tell the transposing LDS reads
// (ds_read_b64_tr_b16) from the loads' destinations, and before each such
// read it would wait for every load in flight (vmcnt(0)), which undoes the
// stage pipeline; the kernel's own vmcnt waits cover these loads as they do
// the builtin's. Wait states: s_nop 4 in case a VALU instruction has just
// written an SGPR the load reads (5 needed), s_nop 0 after writing M0 (1).
template <bool UNTRACKED = false>
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, u32x4 *lds, uint32_t voff,
                                           int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  if constexpr (UNTRACKED) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void *)lds)));
    asm volatile("s_nop 4\n\ts_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(r), "s"(soff)
                 : "m0");
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                             voff, soff, 0, 0);
  }
#endif
}

__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// XOR key of a stage row's 16-byte chunks (rows of 8 chunks)
__device__ __forceinline__ int swz_key(int r) { return r & 7; }
// physical 16-byte chunk of logical chunk c in row r
__device__ __forceinline__ int sw8(int r, int c) { return r * 8 + (c ^ swz_key(r)); }

// K-major B stage buffers: XOR applied to a k-row's chunk-pair index (pairs
// per row a power of two): rows 0-3 and 8-11, 16-19, 24-27 of a k-step (the
// rows one transposing read touches) get distinct values
__device__ __forceinline__ int bkm_swz(int kr, int pairs) {
  return ((kr & 3) | (((kr >> 3) & 3) << 2)) & (pairs - 1);
}

typedef short v4s16 __attribute__((ext_vector_type(4)));

// row (within a 16 x 16 fragment) of accumulator element i of lane `lane`:
// lane (fr, fc) holds rows 4 fc + i of column fr
__device__ __forceinline__ int acc_row(int lane, int i) { return 4 * (lane >> 4) + i; }

// ds_read_b64_tr_b16: within each 16 lanes, lane l receives element l % 4 of
// the 8-byte pieces lanes 4 e + l / 4 point at, e = 0..3 (a 4 x 4 transpose
// of 16-bit elements). (Device-pass only.)
__device__ __forceinline__ v4s16 ds_read_tr16(const char *lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s16 *)(const_cast<char *>(lds)));
#else
  (void)lds;
  return v4s16{0, 0, 0, 0};
#endif
}

// SiLU with the hardware reciprocal (1 ulp) in place of an IEEE division:
// the product is rounded to bf16 or kept in fp32 within the layer's tolerance
__device__ __forceinline__ float silu_f(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0,
                                           static_cast<int>(static_cast<uint32_t>(bytes)),
                                           0x00020000);
}

// LDS of one workgroup: NA A and NA + 1 B stage buffers, reused by the
// epilogue's staging rows; 4-wavefront tiles of at most 80 KB let two
// workgroups share a CU.
template <int BM, int BN, int WGM, int WGN, int NA, int EPI>
struct G2Shape {
  static constexpr int NW = WGM * WGN;
  static constexpr int WTN = BN / WGN;
  static constexpr bool GLU = EPI == EPI_SWIGLU;
  static constexpr int OUTW = GLU ? WTN / 2 : WTN;  // output columns per wave
  static constexpr int PITCH = OUTW + 4;            // floats per staged row
  static constexpr int STAGE16 = (NA * BM + (NA + 1) * BN) * 8;
  static constexpr int STG16 = NW * 16 * PITCH / 4;
  static constexpr int SCL16 = EPI == EPI_SCALE ? BM / 4 : 0;  // row scales after the staging rows
  static constexpr int LDS16 = STAGE16 > STG16 + SCL16 ? STAGE16 : STG16 + SCL16;
  static constexpr int MIN_WAVES = (NW == 4 && LDS16 * 16 <= 80 * 1024) ? 2 : 1;
};

template <int BM, int BN, int WGM, int WGN, int NA, int EPI, bool BKM, bool KS>
__global__ __launch_bounds__(64 * WGM * WGN, (G2Shape<BM, BN, WGM, WGN, NA, EPI>::MIN_WAVES))
void gemm2_kernel(GemmArgs p0, GemmArgs p1) {
  using Sh = G2Shape<BM, BN, WGM, WGN, NA, EPI>;
  constexpr int NB = NA + 1;  // B stage buffers
  static_assert(NA >= 2, "at least double-buffered");
  constexpr int NW = WGM * WGN, THREADS = 64 * NW;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MF = 16;  // fragment edge (v_mfma_f32_16x16x32_bf16)
  constexpr int FM = WTM / MF, FN = WTN / MF;
  constexpr bool GLU = EPI == EPI_SWIGLU;
  constexpr int NOUT = GLU ? BN / 2 : BN;
  constexpr int ROWS = THREADS / 8;                 // rows covered by one load of every thread
  constexpr int A_LD = BM / ROWS, B_LD = BN / ROWS;  // loads per thread per stage
  constexpr int A16 = BM * 8, B16 = BN * 8;          // 16-byte units per stage buffer
  static_assert(BM % ROWS == 0 && BN % ROWS == 0, "whole loads per stage");
  static_assert(!GLU || (BN / 2) % ROWS == 0, "gate and up rows in separate loads");
  static_assert(!GLU || FN % 2 == 0, "paired gate/up fragments");
  static_assert(FM >= 1 && FN >= 1, "at least one fragment per wave");
  static_assert(!(BKM && GLU), "K-major B: no gate/up pairs");
  // K-major B (BKM): B is [K, N] row-major; a stage buffer holds 64 k-rows of
  // BN columns, 16-byte chunks of 8 columns, chunk pairs XOR-swizzled by the
  // k-row so that the 16 rows one transposing read touches fall in distinct
  // banks; fragments are read with ds_read_b64_tr_b16 (4 k-rows x 4 columns
  // per 16 lanes, transposed so each lane holds 4 consecutive k of one
  // column), two reads per 8-k fragment.
  constexpr int KROWB = BN * 2;       // bytes per k-row (BKM)
  constexpr int KPAIRS = BN / 16;     // chunk pairs per k-row (BKM)
  __shared__ __attribute__((aligned(1024))) u32x4 g2_lds[Sh::LDS16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // ------------------------------------------------------------ tile
  // Two problems may share the launch (p1.N == 0: none): the tiles of p0,
  // then those of p1. Consecutive workgroups go to different XCDs: give each
  // XCD a contiguous range of tiles, in groups of m-tiles that run together
  // over all n-tiles so tiles sharing B or A meet in L2.
  // Each problem's tiles are dealt over the XCDs separately (a contiguous
  // range of each per XCD), so two problems of different K balance; the one
  // with the longer reduction runs first on every XCD.
  const int n_tn0 = (p0.N + NOUT - 1) / NOUT;
  const int64_t n_m0 = p0.tiles ? static_cast<int64_t>(*p0.n_tiles) : p0.max_mtiles;
  // (KS, a K-split fp32 store: each tile once per split)
  const int ks0 = KS && p0.k_split > 1 ? p0.k_split : 1;
  const int ks1 = KS && p1.k_split > 1 ? p1.k_split : 1;
  const int64_t total0 = n_m0 * n_tn0 * ks0;
  const int n_tn1 = (p1.N + NOUT - 1) / NOUT;
  const int64_t n_m1 = p1.N <= 0 ? 0 : (p1.tiles ? static_cast<int64_t>(*p1.n_tiles) : p1.max_mtiles);
  const int64_t total1 = n_m1 * n_tn1 * ks1;
  const int64_t per0 = (total0 + 7) / 8, per1 = (total1 + 7) / 8;
  const bool p1_first = total1 > 0 && p1.K + (p1.a2 ? p1.K2 : 0) > p0.K + (p0.a2 ? p0.K2 : 0);
  int64_t local = blockIdx.x >> 3;
  const int xcd = blockIdx.x & 7;
  bool second;
  if (p1_first) {
    second = local < per1;
    if (!second) local -= per1;
  } else {
    second = local >= per0;
    if (second) local -= per0;
  }
  if (local >= (second ? per1 : per0)) return;
  int64_t pid = xcd * (second ? per1 : per0) + local;
  if (pid >= (second ? total1 : total0)) return;
  const GemmArgs &p = second ? p1 : p0;
  const int n_tn = second ? n_tn1 : n_tn0;
  const int64_t n_m = second ? n_m1 : n_m0;
  int split = 0;
  if (KS && (second ? ks1 : ks0) > 1) {  // split-major: all tiles of split 0 first
    const int64_t t2 = n_m * n_tn;
    split = static_cast<int>(pid / t2);
    pid -= split * t2;
  }
  // groups of m-tiles: one expert's (from the table; a group of g m-tiles
  // owns tiles [first n_tn, (first + g) n_tn), so pid / n_tn is one of its
  // m-tiles) or GM consecutive ones (dense); inside a group the m-tile
  // index runs fastest
  constexpr int GM = kGroupM;
  int64_t first_m;
  int gsz;
  if (p.tiles) {
    const int64_t j = pid / n_tn;
    first_m = __builtin_amdgcn_readfirstlane(p.tiles[kTileInts * j + 3]);
    gsz = __builtin_amdgcn_readfirstlane(p.tiles[kTileInts * j + 4]);
  } else {
    first_m = pid / (GM * n_tn) * GM;
    gsz = static_cast<int>(min<int64_t>(n_m - first_m, GM));
  }
  const int64_t in_g = pid - first_m * n_tn;
  const int64_t mt = first_m + in_g % gsz;
  const int nt = static_cast<int>(in_g / gsz);
  int64_t expert = 0, m_begin, m_end;
  if (p.tiles) {
    expert = __builtin_amdgcn_readfirstlane(p.tiles[kTileInts * mt]);
    m_begin = __builtin_amdgcn_readfirstlane(p.tiles[kTileInts * mt + 1]);
    m_end = __builtin_amdgcn_readfirstlane(p.tiles[kTileInts * mt + 2]);
  } else {
    m_begin = mt * BM;
    m_end = min<int64_t>(m_begin + BM, p.M);
  }
  const int n_begin = nt * NOUT;
  // the row-scale epilogue's routing weights, one per tile row: requested
  // before the prologue (loads complete in order, so the stage waits still
  // count right) and parked in LDS after the main loop — a global load per
  // output chunk inside the epilogue cost a dependent load latency in each
  // of its 16-row passes
  float row_w = 1.f;
  if constexpr (EPI == EPI_SCALE) {
    static_assert(64 * WGM * WGN >= BM, "a thread per tile row");
    if (p.row_scale && threadIdx.x < BM && m_begin + threadIdx.x < m_end)
      row_w = p.row_scale[m_begin + threadIdx.x];
  }
  // K-grouped: this expert's reduction columns and output block
  int64_t kbeg = 0, kseg = p.K;
  int64_t obase = 0;
  if (p.k_offsets) {
    kbeg = __builtin_amdgcn_readfirstlane(p.k_offsets[expert]);
    kseg = __builtin_amdgcn_readfirstlane(p.k_offsets[expert + 1]) - kbeg;
    obase = expert * p.out_stride;
  } else if (KS && p.k_split > 1) {  // split s: K columns [s kps, (s + 1) kps), whole stages
    const int64_t kps = ((p.K + 63) / 64 + p.k_split - 1) / p.k_split * 64;
    kbeg = split * kps;
    kseg = min<int64_t>(kps, p.K - kbeg);
    obase = split * p.split_stride;
  }

  // ------------------------------------------------------------ loads
  // load j of a thread: tile row ROWS j + lrow, in the 1 KB block starting at
  // row ROWS j + 8 wave; the slot of lane (lrow, lchunk) holds logical chunk
  // lchunk ^ (lrow & 7)
  const int lrow = tid >> 3;
  const int lchunk = (tid & 7) ^ swz_key(lrow);
  __amdgpu_buffer_rsrc_t ar, br0, br1;
  uint32_t aoff[A_LD];
  uint32_t boff0 = 0, bstep = 0;  // B: row lrow's offset; ROWS rows further (uniform)
  // operand set-up for K segment seg (A and B separately: B is requested a
  // stage further ahead)
  auto setup_a = [&](int seg) {
    if (seg && !p.a2) return;
    const int64_t lda = seg ? p.lda2 : p.lda;
    const int64_t a_rows = seg ? p.M : (p.a_extent ? p.a_extent : p.M);
    ar = rsrc(seg ? p.a2 : p.a, a_rows * lda * 2);
#pragma unroll
    for (int j = 0; j < A_LD; ++j) {
      int64_t m = m_begin + ROWS * j + lrow;
      if (m >= m_end) m = m_begin;
      const int64_t src = (!seg && p.a_rows) ? static_cast<int64_t>(p.a_rows[m]) : m;
      aoff[j] = static_cast<uint32_t>((src * lda + (seg ? 0 : kbeg) + lchunk * 8) * 2);
    }
  };
  uint32_t bkoff[B_LD];  // BKM: each B load's lane offset (stage 0)
  uint32_t bkstage = 0;  // BKM: bytes per stage (64 k-rows)
  auto setup_b = [&](int seg) {
    if (seg && !p.a2) return;
    if constexpr (BKM) {
      const int64_t ldb = seg ? p.ldb2 : p.ldb;
      const int64_t kseg_b = seg ? p.K2 : kseg;
      const int64_t bytes = kseg_b * ldb * 2;
      const int64_t eoff = expert * (seg ? p.b2_stride : p.b_stride) * 2;
      br0 = br1 = rsrc(static_cast<const char *>(seg ? p.b2 : p.b0) + eoff, bytes);
#pragma unroll
      for (int j = 0; j < B_LD; ++j) {
        // byte o of the stage buffer: k-row o / KROWB, physical chunk
        // (o % KROWB) / 16, holding logical chunk pair (pc / 2) ^ swizzle
        const int o = (NW * j + wave) * 1024 + lane * 16;
        const int kr = o / KROWB, pc = (o % KROWB) / 16;
        const int lc = (((pc >> 1) ^ bkm_swz(kr, KPAIRS)) << 1) | (pc & 1);
        bkoff[j] = static_cast<uint32_t>((kr * ldb + n_begin + lc * 8) * 2);
      }
      bkstage = static_cast<uint32_t>(64 * ldb * 2);
      return;
    }
    const int64_t ldb = seg ? p.ldb2 : p.ldb, bytes = static_cast<int64_t>(p.N) * ldb * 2;
    if (seg) {
      br0 = br1 = rsrc(static_cast<const char *>(p.b2) + expert * p.b2_stride * 2, bytes);
    } else {
      const int64_t eoff = expert * p.b_stride * 2;
      br0 = rsrc(static_cast<const char *>(p.b0) + eoff, bytes);
      br1 = GLU ? rsrc(static_cast<const char *>(p.b1) + eoff, bytes) : br0;
    }
    boff0 = static_cast<uint32_t>(
        (static_cast<int64_t>(n_begin + lrow) * ldb + (seg ? 0 : kbeg) + lchunk * 8) * 2);
    bstep = static_cast<uint32_t>(ROWS * ldb * 2);
  };

  // a last K segment that ends 32 columns into a stage runs only that
  // stage's first k-step (the other half of its buffers holds columns past
  // the row: the next row's, or zeros past the operand's extent)
  const int steps1 = static_cast<int>((kseg + 63) / 64);
  const int steps = steps1 + (p.a2 ? (p.K2 + 63) / 64 : 0);
  const int last = steps - 1;
  const bool half_last = ((p.a2 ? p.K2 : kseg) & 63) != 0;
  auto kbytes = [&](int st) {
    return __builtin_amdgcn_readfirstlane((st >= steps1 ? st - steps1 : st) * kRowBytes);
  };
  auto load_a = [&](u32x4 *ab, int st, int j) {
    load_lds16<BKM>(ar, ab + (ROWS * j + 8 * wave) * 8, aoff[j], kbytes(st));
  };
  auto load_b = [&](u32x4 *bb, int st, int j) {
    if constexpr (BKM) {
      const int sl = st >= steps1 ? st - steps1 : st;
      load_lds16<BKM>(br0, bb + (NW * j + wave) * 64, bkoff[j],
                 __builtin_amdgcn_readfirstlane(sl * bkstage));
      return;
    }
    const bool up = GLU && j >= B_LD / 2;  // gate rows first, then up rows
    load_lds16<BKM>(up ? br1 : br0, bb + (ROWS * j + 8 * wave) * 8,
               boff0 + (up ? j - B_LD / 2 : j) * bstep, kbytes(st));
  };

  // ------------------------------------------------------------ fragments
  const int fr = lane & 15, fc = lane >> 4;
  auto brow_of = [&](int fn) {  // B row (within the tile) of fragment fn
    if (GLU) {
      constexpr int half = FN / 2;
      return fn < half ? wn * (WTN / 2) + fn * MF : BN / 2 + wn * (WTN / 2) + (fn - half) * MF;
    }
    return wn * WTN + fn * MF;
  };
  // this wave's 16-row fragments that hold rows of the tile
  // fragment row fm of wavefront row wm holds tile rows frow(fm) .. + MF - 1:
  // interleaved over the wavefront rows (fm WGM + wm), so that a tile with
  // fewer rows than BM spreads its MFMAs over all four SIMDs (two wavefront
  // rows share a SIMD) instead of leaving the SIMDs of the last rows idle
  auto frow = [&](int fm) { return (fm * WGM + wm) * MF; };
  const int64_t rows_in = m_end - m_begin;
  const int64_t n_frag = (rows_in + MF - 1) / MF;  // fragment rows holding tile rows
  const int live = __builtin_amdgcn_readfirstlane(
      static_cast<int>(min<int64_t>(FM, max<int64_t>(0, (n_frag - wm + WGM - 1) / WGM))));

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 *const abuf = g2_lds;             // A: NA x A16
  u32x4 *const bbuf = g2_lds + NA * A16;  // B: NB x B16
  // per 32-k step a fragment takes one 16-byte read per lane (lane (fr, fc):
  // row fr, 8 k at 8 fc)
  bf16x8 xa0[FM], xb0[FN], xa1[FM], xb1[FN];
  auto rd = [&](const u32x4 *ab, const u32x4 *bb, int ks, int i, bf16x8 *xa, bf16x8 *xb) {
    const int kc = 4 * ks + fc;
    if (i < FN) {
      if constexpr (BKM) {
        // lane (g = lane / 16, r = (lane % 16) / 4, q = lane % 4) points at
        // k-row 32 ks + 8 g + 4 h + r, columns brow + 4 q .. + 3; the
        // transposing read hands lane l the 4 k of column brow + l % 16
        const int g = lane >> 4, r = (lane >> 2) & 3, q = lane & 3;
        const int lc = (brow_of(i) >> 3) + (q >> 1);
        const char *base = reinterpret_cast<const char *>(bb);
        v4s16 h2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int kr = 32 * ks + 8 * g + 4 * h + r;
          const int pc = (((lc >> 1) ^ bkm_swz(kr, KPAIRS)) << 1) | (lc & 1);
          h2[h] = ds_read_tr16(base + kr * KROWB + pc * 16 + (q & 1) * 8);
        }
        xb[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h2[0], h2[1], 0, 1, 2, 3, 4, 5,
                                                                   6, 7));
      } else {
        xb[i] = __builtin_bit_cast(bf16x8, bb[sw8(brow_of(i) + fr, kc)]);
      }
    } else
      xa[i - FN] = __builtin_bit_cast(bf16x8, ab[sw8(frow(i - FN) + fr, kc)]);
  };
  auto mrow = [&](int fm, const bf16x8 *xa, const bf16x8 *xb) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
      acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[fm], xb[fn], acc[fm][fn], 0, 0, 0);
  };
  constexpr int NRD = FM + FN;                         // fragment reads per set
  constexpr int RD_PER = (NRD + FM - 1) / FM;          // ... per MFMA row
  constexpr int LD_PER = (A_LD + B_LD + FM - 1) / FM;  // loads per MFMA row

  // ------------------------------------------------------------ main loop
  // (each operand switches to the second K segment's rows before its first
  // load from that segment; loads are issued in stage order per operand)
  setup_a(0);
  setup_b(0);
  auto seg_a = [&](int st) {
    if (st == steps1) setup_a(1);
  };
  auto seg_b = [&](int st) {
    if (st == steps1) setup_b(1);
  };
  // prologue: A(0..NA-1) and B(0..NB-1), interleaved in stage order
#pragma unroll
  for (int s0 = 0; s0 < NB; ++s0) {
    const int sl = min(s0, last);
    if (s0 < NA) {
      seg_a(sl);
#pragma unroll
      for (int j = 0; j < A_LD; ++j) load_a(abuf + s0 * A16, sl, j);
    }
    seg_b(sl);
#pragma unroll
    for (int j = 0; j < B_LD; ++j) load_b(bbuf + s0 * B16, sl, j);
  }
  wait_vm_lgkm0<(NA - 1) * A_LD + (NB - 1) * B_LD>();  // stage 0 has landed
  barrier();
#pragma unroll
  for (int i = 0; i < NRD; ++i) rd(abuf, bbuf, 0, i, xa0, xb0);

  // the K loop issues at wave priority 1: a co-resident workgroup's prologue
  // or epilogue yields to it (measured: large prefill -0.8%, others level)
  __builtin_amdgcn_s_setprio(1);
  int a_cur = 0, b_cur = 0;  // st % NA, st % NB
  for (int st = 0; st < steps; ++st) {
    const int a_nxt = a_cur == NA - 1 ? 0 : a_cur + 1;
    const int b_nxt = b_cur == NB - 1 ? 0 : b_cur + 1;
    u32x4 *const ac = abuf + a_cur * A16, *const an = abuf + a_nxt * A16;
    u32x4 *const bc = bbuf + b_cur * B16, *const bn = bbuf + b_nxt * B16;
    wait_lgkm0();  // set 0 has landed
    // per fragment row: the LDS reads for the next k-step go out before the
    // row's MFMAs, so the last reads' latency overlaps the last MFMAs
    // (measured: small -1.3%, latent -0.8%, large prefill -0.8%)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
      for (int q = 0; q < RD_PER; ++q) {
        const int i = fm * RD_PER + q;
        if (i < NRD) rd(ac, bc, 1, i, xa1, xb1);
      }
      if (fm < live) mrow(fm, xa0, xb0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // A and B of st + 1 have landed (the loads issued after them: the B
    // half of A(st + 1)'s batch and NA - 2 full batches)
    wait_vm_lgkm0<(NA - 2) * A_LD + (NB - 2) * B_LD>();
    barrier();
    const int sa = min(st + NA, last), sb = min(st + NB, last);
    if (st + NA <= last) seg_a(sa);
    if (st + NB <= last) seg_b(sb);
    const int live1 = (half_last && st == last) ? 0 : live;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
      for (int q = 0; q < RD_PER; ++q) {
        const int i = fm * RD_PER + q;
        if (i < NRD) rd(an, bn, 0, i, xa0, xb0);
      }
      if (fm < live1) mrow(fm, xa1, xb1);
#pragma unroll
      for (int q = 0; q < LD_PER; ++q) {
        const int j = fm * LD_PER + q;
        if (j < A_LD) load_a(ac, sa, j);
        else if (j < A_LD + B_LD) load_b(bc, sb, j - A_LD);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    a_cur = a_nxt;
    b_cur = b_nxt;
  }
  __builtin_amdgcn_s_setprio(0);
  wait_vm_lgkm0<0>();
  barrier();  // the epilogue reuses the stage buffers
  float *const row_scale_lds = reinterpret_cast<float *>(g2_lds) + Sh::STG16 * 4;
  if constexpr (EPI == EPI_SCALE) {
    if (tid < BM) row_scale_lds[tid] = row_w;
    barrier();
  }

  // ------------------------------------------------------------ epilogue
  if constexpr (EPI == EPI_STORE_F32) {
    // fp32 out straight from the accumulators: lane (fr, fc) holds rows
    // 4 fc + i, column fr of each 16x16 fragment, so each store writes four
    // 64-byte row pieces (measured 1-2% faster on the backward's fp32
    // products than staging through LDS). One row address per (fragment
    // row, i); the fragments of a row are immediate offsets from it. Tiles
    // wholly inside the output store without per-element checks.
    const int64_t ldo = p.ldo;
    const int col_l = wn * WTN + (lane % MF);  // this lane's column within the tile
    float *const o_l = static_cast<float *>(p.out) + obase + (m_begin + acc_row(lane, 0)) * ldo +
                       n_begin + col_l;
    if (rows_in >= BM && n_begin + BN <= p.N) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float *const orow = o_l + static_cast<int64_t>(frow(fm) + i) * ldo;
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) orow[fn * MF] = acc[fm][fn][i];
        }
      return;
    }
    const int rows32 = static_cast<int>(rows_in), cols_in = p.N - n_begin - col_l;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if (fm >= live) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (frow(fm) + acc_row(lane, i) >= rows32) continue;
        float *const orow = o_l + static_cast<int64_t>(frow(fm) + i) * ldo;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          if (fn * MF < cols_in) orow[fn * MF] = acc[fm][fn][i];
      }
    }
    return;
  }
  // each wave: 16 rows x OUTW columns of fp32 at a time in its own slice
  constexpr int OUTW = Sh::OUTW;
  constexpr int FO = GLU ? FN / 2 : FN;
  constexpr int PITCH = Sh::PITCH;
  float *stg = reinterpret_cast<float *>(g2_lds) + wave * 16 * PITCH;
  const int col0 = n_begin + (GLU ? wn * (WTN / 2) : wn * WTN);
  // each lane stores one 8-column chunk of rows r0, r0 + RSTEP, ... of a
  // 16-row pass: its column (and column bound) is fixed, its output address
  // steps one uniform row stride per item
  constexpr int CPR8 = OUTW / 8;  // 8-column chunks per staged row
  static_assert(64 % CPR8 == 0, "whole rows per 64 lanes");
  constexpr int RSTEP = 64 / CPR8, NIT = (16 + RSTEP - 1) / RSTEP;
  const int c8 = (lane % CPR8) * 8, r0 = lane / CPR8;
  const int col = col0 + c8;
  const bool col_ok = col < p.N;
  const int rows32 = static_cast<int>(rows_in);
  const bool f32o = EPI == EPI_STORE_F32 || (EPI == EPI_SCALE && p.out_f32);
  const int64_t esz = f32o ? 4 : 2;
  char *const obytes = static_cast<char *>(p.out) + (obase + m_begin * p.ldo + col) * esz;
  const int64_t rstride = p.ldo * esz;
  // one pass per fragment row (16 rows)
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    if (fm >= live) break;  // unrolled: acc is indexed statically and stays in registers
#pragma unroll
    for (int fo = 0; fo < FO; ++fo)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = acc[fm][fo][i];
        if (GLU) v = silu_f(v) * acc[fm][fo + FO][i];
        stg[acc_row(lane, i) * PITCH + fo * MF + (lane % MF)] = v;
      }
    __builtin_amdgcn_s_waitcnt(0xC07F & ~0x0F00);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    const int rel0 = frow(fm) + r0;  // tile row of item 0
    // the pass's LDS reads all go out first (a row past the 16 staged ones
    // reads row 15 and is never stored), then the items are scaled,
    // converted and stored (the row weights are 1 where none are given, so
    // the scaling needs no branch)
    float v[NIT][8], sc[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int r = min(r0 + it * RSTEP, 15);
      const float4 lo = *reinterpret_cast<const float4 *>(stg + r * PITCH + c8);
      const float4 hi = *reinterpret_cast<const float4 *>(stg + r * PITCH + c8 + 4);
      v[it][0] = lo.x; v[it][1] = lo.y; v[it][2] = lo.z; v[it][3] = lo.w;
      v[it][4] = hi.x; v[it][5] = hi.y; v[it][6] = hi.z; v[it][7] = hi.w;
      sc[it] = EPI == EPI_SCALE ? row_scale_lds[min(rel0 + it * RSTEP, BM - 1)] : 1.f;
    }
    auto store_items = [&](auto f32_c) {
      constexpr bool F32 = decltype(f32_c)::value;
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int r = r0 + it * RSTEP, rel = rel0 + it * RSTEP;
        if ((RSTEP > 16 && r >= 16) || !col_ok || rel >= rows32) continue;
        float *const w = v[it];
        if (EPI == EPI_SCALE) {
#pragma unroll
          for (int q = 0; q < 8; ++q) w[q] *= sc[it];
        }
        if (EPI == EPI_COMBINE) {
          const int64_t m = m_begin + rel;
          float rs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          for (int k = 0; k < p.topk; ++k) {
            const int q = p.inv[m * p.topk + k];
            if (q < 0) continue;
            float y[8];
            Chunk<bf16_t>::unpack(*reinterpret_cast<const uint4 *>(
                                      static_cast<const uint16_t *>(p.y) + static_cast<int64_t>(q) * p.ldy + col),
                                  y);
#pragma unroll
            for (int e = 0; e < 8; ++e) rs[e] += y[e];
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] += rs[e];
        }
        char *const o = obytes + rel * rstride;
        if constexpr (F32) {
          reinterpret_cast<float4 *>(o)[0] = make_float4(w[0], w[1], w[2], w[3]);
          reinterpret_cast<float4 *>(o)[1] = make_float4(w[4], w[5], w[6], w[7]);
        } else {
          *reinterpret_cast<uint4 *>(o) = Chunk<bf16_t>::pack(w);
        }
      }
    };
    if (f32o)
      store_items(std::true_type{});
    else
      store_items(std::false_type{});
    __builtin_amdgcn_s_waitcnt(0xC07F & ~0x0F00);  // lgkmcnt(0): reads done before rewrite
    asm volatile("" ::: "memory");
  }
}

typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef int v4i32 __attribute__((ext_vector_type(4)));

// Value of lane 16 (l / 16) + I for each lane l (within each 16-lane row:
// its lane I), by a bit-mode swizzle (source lane (l & 16) | I of each 32).
template <int I>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x10 | (I << 5)));
}

// ------------------------------------------------------------------ persistent
// Persistent form of the 256x256 tile (4 x 2 wavefronts of 64x128, A two
// stages ahead) for one problem (no second K segment or K split; K-grouped
// allowed) and an epilogue that writes from the accumulators: SwiGLU, row
// scale, fp32 store, or the gate and up halves of a SwiGLU tile each stored
// in fp32 (the backward's recomputed pre-activations). Each workgroup runs a
// fixed list of tiles:
// the tiles are dealt over the XCDs in contiguous ranges as in gemm2_kernel,
// and workgroup w of an XCD takes tiles w, w + G, w + 2 G, ... of its range
// (G workgroups per XCD), so that at any time an XCD works on G consecutive
// tiles and tiles sharing operands still meet in L2.
//
// The stage pipeline runs on across tiles: the loads a tile's last stages
// would spend on repeats of its last stage fetch the next tile's first
// stages instead (B from three stages before the end, A from two), and the
// fragment reads at the end of a tile's last stage are the next tile's
// first. The epilogue then needs no LDS (every stage buffer holds the next
// tile's data): B rows are loaded in an order that gives each lane a run of
// adjacent output columns, RUN = 8 (4 for SwiGLU, whose gate and up
// fragments pair up), so it stores straight from its accumulators, one
// 16-byte (8-byte) piece per row. The next tile is decoded during the
// current one's first stages (the tile table, then the expert's reduction
// range: dependent reads a stage apart, their latency under MFMAs); its A
// rows are gathered once the current tile's last A loads are out and become
// offsets a stage later. The epilogue's stores are waited for by the next
// tile's first stage wait. A tile of fewer than 5 stages, or followed by one
// of fewer than 3, drains its loads instead, and the next tile starts with
// a prologue of its own (a K-grouped expert without reduction columns runs
// no stages: its output is zeros).
//
// Lane (fr, fc) holds rows 4 fc + i of column fr of each 16 x 16 fragment.
// Stage buffer row R of B holds, within each 128-row block (64 for each of
// SwiGLU's gate and up halves) of fragments f = (R % 128) / 16, lanes
// fr = R % 16, the weight row of output column RUN fr + f of the block.
template <int EPI>
__global__ __launch_bounds__(512, 1) void gemm2p_kernel(GemmArgs p) {
  constexpr int BM = 256, BN = 256, WGM = 4, WGN = 2, NA = 2, NB = NA + 1;
  constexpr int NW = WGM * WGN, THREADS = 64 * NW;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MF = 16, FM = WTM / MF, FN = WTN / MF;
  constexpr bool GLU = EPI == EPI_SWIGLU || EPI == EPI_GLU_F32;  // gate and up halves
  constexpr int NOUT = GLU ? BN / 2 : BN;
  constexpr int ROWS = THREADS / 8, A_LD = BM / ROWS, B_LD = BN / ROWS;
  constexpr int A16 = BM * 8, B16 = BN * 8;
  constexpr int RUN = GLU ? FN / 2 : FN;  // adjacent output columns per lane
  static_assert(EPI == EPI_SWIGLU || EPI == EPI_SCALE || EPI == EPI_STORE_F32 ||
                    EPI == EPI_GLU_F32,
                "epilogues that store from the accumulators");
  static_assert(A_LD == 4 && B_LD == 4 && FM == 4 && FN == 8, "tile geometry");
  __shared__ __attribute__((aligned(1024))) u32x4 g2p_lds[(NA * BM + NB * BN) * 8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // (uniform: scalar arithmetic)
  // the thread index, opaque: lane-dependent values used once per tile are
  // formed from it where they are used, not held across the K loop
  auto tid_o = [&]() {
    int t = tid;
    asm volatile("" : "+v"(t));
    return t;
  };
  const int wm = wave / WGN, wn = wave % WGN;
  const int fr = lane & 15, fc = lane >> 4;

  // ------------------------------------------------------------ tile list
  // (tile counts, rows and columns fit 32 bits: the host bounds the
  // operands' byte extents below 4 GiB)
  const int n_tn = (p.N + NOUT - 1) / NOUT;
  const int n_m = p.tiles ? *p.n_tiles : static_cast<int>(p.max_mtiles);
  const int total = n_m * n_tn, per = (total + 7) / 8;
  const int xcd = blockIdx.x & 7, gstride = gridDim.x >> 3;
  const int t_end = min(total, (xcd + 1) * per);
  int pid = xcd * per + (blockIdx.x >> 3);
  if (pid >= t_end) return;

  // tile decode in two steps (its group of m-tiles; then its table entry),
  // so that the dependent table reads can sit half a stage apart
  constexpr int GM = kGroupM;
  // (read as constant memory: scalar loads, which the stage waits do not count)
  const __attribute__((address_space(4))) int32_t *const tt =
      (const __attribute__((address_space(4))) int32_t *)p.tiles;
  auto group_of = [&](int q, int &first_m, int &gsz) {
    if (p.tiles) {
      const int j = q / n_tn;
      first_m = __builtin_amdgcn_readfirstlane(tt[kTileInts * j + 3]);
      gsz = __builtin_amdgcn_readfirstlane(tt[kTileInts * j + 4]);
    } else {
      first_m = q / (GM * n_tn) * GM;
      gsz = min(n_m - first_m, GM);
    }
  };
  auto tile_of = [&](int q, int first_m, int gsz, int &expert, int &m_begin, int &m_end,
                     int &n_begin) {
    const int in_g = q - first_m * n_tn;
    const int mt = first_m + in_g % gsz;
    n_begin = (in_g / gsz) * NOUT;
    if (p.tiles) {
      expert = __builtin_amdgcn_readfirstlane(tt[kTileInts * mt]);
      m_begin = __builtin_amdgcn_readfirstlane(tt[kTileInts * mt + 1]);
      m_end = __builtin_amdgcn_readfirstlane(tt[kTileInts * mt + 2]);
    } else {
      expert = 0;
      m_begin = mt * BM;
      m_end = static_cast<int>(min<int64_t>(m_begin + BM, p.M));
    }
  };
  // K-grouped: the expert's reduction columns [kbeg, kbeg + kseg) (a
  // multiple of 64; 0 for an expert with no rows: its output is zeros)
  const __attribute__((address_space(4))) int32_t *const ko =
      (const __attribute__((address_space(4))) int32_t *)p.k_offsets;
  auto k_of = [&](int expert, int &kbeg, int &kseg) {
    if (p.k_offsets) {
      kbeg = __builtin_amdgcn_readfirstlane(ko[expert]);
      kseg = __builtin_amdgcn_readfirstlane(ko[expert + 1]) - kbeg;
    } else {
      kbeg = 0;
      kseg = p.K;
    }
  };
  // fragment row fm of wavefront row wm holds tile rows frow(fm) .. + 15
  // (interleaved over the wavefront rows as in gemm2_kernel); live: the
  // fragment rows that hold tile rows
  auto frow = [&](int fm) { return (fm * WGM + wm) * MF; };
  auto live_of = [&](int rows_in) {
    const int n_frag = (rows_in + MF - 1) / MF;
    return __builtin_amdgcn_readfirstlane(min(FM, max(0, (n_frag - wm + WGM - 1) / WGM)));
  };

  // ------------------------------------------------------------ loads
  // load j of a thread: stage row ROWS j + lrow (A: tile row; B: see above),
  // in the 1 KB block at row ROWS j + 8 wave, logical chunk lchunk
  auto lrow_of = [&](int t) { return t >> 3; };
  auto lchunk_of = [&](int t) { return (t & 7) ^ swz_key(t >> 3); };
  const uint32_t arow_bytes = static_cast<uint32_t>(p.lda * 2);
  const uint32_t brow_bytes = static_cast<uint32_t>(p.ldb * 2);
  const int64_t a_rows_ext = p.a_extent ? p.a_extent : p.M;
  const __amdgpu_buffer_rsrc_t ar = rsrc(p.a, a_rows_ext * p.lda * 2);
  // B: the weight row of stage row ROWS j + lrow is n_begin + bperm + bj(j)
  auto bperm_of = [&](int lrow) {
    return GLU ? (lrow % 16) * 4 + lrow / 16 : (lrow % 16) * 8 + lrow / 16;
  };
  auto bj = [&](int j) { return GLU ? (j % 2) * 64 : (j / 2) * 128 + (j % 2) * 4; };
  const int64_t b_bytes = static_cast<int64_t>(p.N) * p.ldb * 2;
  __amdgpu_buffer_rsrc_t br0, br1;
  uint32_t boff = 0;
  auto b_setup = [&](int expert, int n_begin, int kbeg) {
    const int64_t eoff = static_cast<int64_t>(expert) * p.b_stride * 2;
    br0 = rsrc(static_cast<const char *>(p.b0) + eoff, b_bytes);
    br1 = GLU ? rsrc(static_cast<const char *>(p.b1) + eoff, b_bytes) : br0;
    const int t = tid_o();
    boff = static_cast<uint32_t>(n_begin + bperm_of(lrow_of(t))) * brow_bytes +
           (kbeg + lchunk_of(t) * 8) * 2;
  };
  // A rows of the tile's loads (gathered rows when given; rows past the
  // tile's end repeat its first row), then, in place, their offsets
  // (the gather through a buffer resource: 32-bit lane offsets; every
  // index read is below m_end)
  uint32_t aoff[A_LD];
  const __amdgpu_buffer_rsrc_t gr = rsrc(p.a_rows, p.a_rows ? 0xFFFFFFFFll : 0);
  auto a_gather = [&](int m_begin, int m_end) {
#pragma unroll
    for (int j = 0; j < A_LD; ++j) {
      int m = m_begin + ROWS * j + lrow_of(tid_o());
      if (m >= m_end) m = m_begin;
      aoff[j] = p.a_rows ? __builtin_amdgcn_raw_buffer_load_b32(gr, m * 4, 0, 0)
                         : static_cast<uint32_t>(m);
    }
  };
  auto a_offsets = [&](int kbeg) {
#pragma unroll
    for (int j = 0; j < A_LD; ++j)
      aoff[j] = aoff[j] * arow_bytes + (kbeg + lchunk_of(tid_o()) * 8) * 2;
  };
  auto load_a = [&](u32x4 *ab, int st, int j) {
    load_lds16(ar, ab + (ROWS * j + 8 * wave) * 8, aoff[j],
               __builtin_amdgcn_readfirstlane(st * kRowBytes));
  };
  auto load_b = [&](u32x4 *bb, int st, int j) {
    const bool up = GLU && j >= B_LD / 2;
    load_lds16(up ? br1 : br0, bb + (ROWS * j + 8 * wave) * 8, boff + bj(j) * brow_bytes,
               __builtin_amdgcn_readfirstlane(st * kRowBytes));
  };

  // ------------------------------------------------------------ fragments
  auto brow_of = [&](int fn) {  // B stage row (within the tile) of fragment fn
    if (GLU) {
      constexpr int half = FN / 2;
      return fn < half ? wn * (WTN / 2) + fn * MF : BN / 2 + wn * (WTN / 2) + (fn - half) * MF;
    }
    return wn * WTN + fn * MF;
  };
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 *const abuf = g2p_lds;
  u32x4 *const bbuf = g2p_lds + NA * A16;
  bf16x8 xa0[FM], xb0[FN], xa1[FM], xb1[FN];
  auto rd = [&](const u32x4 *ab, const u32x4 *bb, int ks, int i, bf16x8 *xa, bf16x8 *xb) {
    const int kc = 4 * ks + fc;
    if (i < FN)
      xb[i] = __builtin_bit_cast(bf16x8, bb[sw8(brow_of(i) + fr, kc)]);
    else
      xa[i - FN] = __builtin_bit_cast(bf16x8, ab[sw8(frow(i - FN) + fr, kc)]);
  };
  auto mrow = [&](int fm, const bf16x8 *xa, const bf16x8 *xb) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
      acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[fm], xb[fn], acc[fm][fn], 0, 0, 0);
  };
  constexpr int NRD = FM + FN;
  constexpr int RD_PER = (NRD + FM - 1) / FM;
  constexpr int LD_PER = (A_LD + B_LD + FM - 1) / FM;

  // ------------------------------------------------------------ epilogue
  // row scales: lane (r, c) of 16-lane row c holds the weight of tile row
  // frow(fm) + 4 c + (r & 3); row_bcast hands each lane the one of its row
  const __amdgpu_buffer_rsrc_t sr =
      rsrc(p.row_scale, (EPI == EPI_SCALE && p.row_scale ? a_rows_ext : 0) * 4);
  float wsc[FM];
  auto scale_load = [&](int m_begin) {
    if constexpr (EPI == EPI_SCALE) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int t = tid_o();
        const int r = m_begin + frow(fm) + 4 * ((t & 63) >> 4) + (t & 3);
        wsc[fm] = p.row_scale ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                             sr, r * 4, 0, 0))
                              : 1.f;
      }
    }
  };
  // stores through a buffer resource at the tile's first row: one lane
  // offset (its rows 4 fc, its run's column), a uniform row offset per
  // fragment row and element
  auto epilogue = [&](int m_begin, int rows_in, int n_begin, int expert, int live) {
    // (N is a multiple of 8: a lane's run is wholly in or out)
    const int t = tid_o();
    const int col = n_begin + wn * (WTN / (GLU ? 2 : 1)) + (t & 15) * RUN;
    const bool col_ok = col < p.N;
    const bool f32o =
        EPI == EPI_STORE_F32 || EPI == EPI_GLU_F32 || (EPI == EPI_SCALE && p.out_f32);
    const int esz = f32o ? 4 : 2;
    // (opaque here, so that the row offsets and row checks below are formed
    // per tile, not held across the K loop)
    uint32_t rbytes = static_cast<uint32_t>(p.ldo) * esz;
    int lane_row = 4 * ((t & 63) >> 4);
    asm volatile("" : "+s"(rbytes));
    asm volatile("" : "+v"(lane_row));
    const int64_t obase = p.k_offsets ? static_cast<int64_t>(expert) * p.out_stride : 0;
    const __amdgpu_buffer_rsrc_t orr =
        rsrc(static_cast<char *>(p.out) + (obase + static_cast<int64_t>(m_begin) * p.ldo) * esz,
             static_cast<int64_t>(rows_in) * rbytes);
    const __amdgpu_buffer_rsrc_t orr2 =
        EPI == EPI_GLU_F32
            ? rsrc(static_cast<char *>(p.out2) + static_cast<int64_t>(m_begin) * p.ldo * esz,
                   static_cast<int64_t>(rows_in) * rbytes)
            : orr;
    const int voff = static_cast<int>(lane_row * rbytes + col * esz);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if (fm >= live) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = frow(fm) + i;  // + lane_row
        float v[RUN];
        if constexpr (EPI == EPI_GLU_F32) {
#pragma unroll
          for (int q = 0; q < RUN; ++q) v[q] = acc[fm][q][i];
        } else if constexpr (GLU) {
#pragma unroll
          for (int q = 0; q < RUN; ++q) v[q] = silu_f(acc[fm][q][i]) * acc[fm][q + RUN][i];
        } else {
#pragma unroll
          for (int q = 0; q < RUN; ++q) v[q] = acc[fm][q][i];
        }
        if constexpr (EPI == EPI_SCALE) {
          const float w = i == 0 ? row_bcast<0>(wsc[fm])
                        : i == 1 ? row_bcast<1>(wsc[fm])
                        : i == 2 ? row_bcast<2>(wsc[fm])
                                 : row_bcast<3>(wsc[fm]);
#pragma unroll
          for (int q = 0; q < RUN; ++q) v[q] *= w;
        }
        // (after the swizzle: every lane takes part in it)
        if (!col_ok || lane_row >= rows_in - r) continue;
        const int so =
            __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(r) * rbytes));
        if constexpr (EPI == EPI_GLU_F32) {
          const v4i32 dg = {__float_as_int(v[0]), __float_as_int(v[1]), __float_as_int(v[2]),
                            __float_as_int(v[3])};
          const v4i32 du = {__float_as_int(acc[fm][RUN][i]), __float_as_int(acc[fm][RUN + 1][i]),
                            __float_as_int(acc[fm][RUN + 2][i]),
                            __float_as_int(acc[fm][RUN + 3][i])};
          __builtin_amdgcn_raw_buffer_store_b128(dg, orr, voff, so, 0);
          __builtin_amdgcn_raw_buffer_store_b128(du, orr2, voff, so, 0);
        } else if constexpr (GLU) {
          const v2i32 d = {static_cast<int>(f32x2_to_bf16x2(v[0], v[1])),
                           static_cast<int>(f32x2_to_bf16x2(v[2], v[3]))};
          __builtin_amdgcn_raw_buffer_store_b64(d, orr, voff, so, 0);
        } else if (f32o) {
          const v4i32 d0 = {__float_as_int(v[0]), __float_as_int(v[1]), __float_as_int(v[2]),
                            __float_as_int(v[3])};
          const v4i32 d1 = {__float_as_int(v[4]), __float_as_int(v[5]), __float_as_int(v[6]),
                            __float_as_int(v[7])};
          __builtin_amdgcn_raw_buffer_store_b128(d0, orr, voff, so, 0);
          __builtin_amdgcn_raw_buffer_store_b128(d1, orr, voff + 16, so, 0);
        } else {
          const uint4 c = Chunk<bf16_t>::pack(v);
          const v4i32 d = {static_cast<int>(c.x), static_cast<int>(c.y), static_cast<int>(c.z),
                           static_cast<int>(c.w)};
          __builtin_amdgcn_raw_buffer_store_b128(d, orr, voff, so, 0);
        }
        // one row at a time: the next tile's first fragments stay live
        // across the epilogue, which leaves it few registers
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ------------------------------------------------------------ tiles
  // A tile whose next one has at least NB stages, and which itself has at
  // least 5 (its stages 0 - 2 decode the next tile), fetches the next tile's
  // first stages in its own last ones ("primes" it); any other tile drains
  // its loads and the next one starts with a prologue of its own.
  auto n_stages = [&](int kseg) { return (kseg + 63) / 64; };
  int c_mb, c_me, c_nb, c_exp, c_kb = 0, c_ks = p.K;
  {
    int first_m, gsz;
    group_of(pid, first_m, gsz);
    tile_of(pid, first_m, gsz, c_exp, c_mb, c_me, c_nb);
    k_of(c_exp, c_kb, c_ks);
  }
  bool primed = false;
  int a_cur = 0, b_cur = 0;
  while (true) {
    const int steps = n_stages(c_ks), last = steps - 1;
    const bool half_last = (c_ks & 63) != 0;
    const int c_live = live_of(c_me - c_mb);
    if (!primed) {
      // the previous tile's loads have landed and its reads are done
      wait_vm_lgkm0<0>();
      barrier();
      a_cur = b_cur = 0;
      if (steps > 0) {
        b_setup(c_exp, c_nb, c_kb);
        a_gather(c_mb, c_me);
        a_offsets(c_kb);
#pragma unroll
        for (int s0 = 0; s0 < NB; ++s0) {
          if (s0 < NA) {
#pragma unroll
            for (int j = 0; j < A_LD; ++j) load_a(abuf + s0 * A16, min(s0, last), j);
          }
#pragma unroll
          for (int j = 0; j < B_LD; ++j) load_b(bbuf + s0 * B16, min(s0, last), j);
        }
        wait_vm_lgkm0<(NA - 1) * A_LD + (NB - 1) * B_LD>();
        barrier();
#pragma unroll
        for (int i = 0; i < NRD; ++i) rd(abuf, bbuf, 0, i, xa0, xb0);
      }
    }
    const int n_pid = pid + gstride;
    const bool n_ok = n_pid < t_end;  // there is a next tile
    int n_first = 0, n_gsz = 1, n_exp = 0, n_mb = 0, n_me = 0, n_nb = 0, n_kb = 0, n_ks = p.K;
    bool pf = false;  // this tile primes the next
    __builtin_amdgcn_s_setprio(1);
    for (int st = 0; st < steps; ++st) {
      const int a_nxt = a_cur == NA - 1 ? 0 : a_cur + 1;
      const int b_nxt = b_cur == NB - 1 ? 0 : b_cur + 1;
      u32x4 *const ac = abuf + a_cur * A16, *const an = abuf + a_nxt * A16;
      u32x4 *const bc = bbuf + b_cur * B16, *const bn = bbuf + b_nxt * B16;
      wait_lgkm0();
      if (st == 0 && n_ok && steps >= 5) group_of(n_pid, n_first, n_gsz);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int q = 0; q < RD_PER; ++q) {
          const int i = fm * RD_PER + q;
          if (i < NRD) rd(ac, bc, 1, i, xa1, xb1);
        }
        if (fm < c_live) mrow(fm, xa0, xb0);
        __builtin_amdgcn_sched_barrier(0);
      }
      wait_vm_lgkm0<(NA - 2) * A_LD + (NB - 2) * B_LD>();
      barrier();
      if (st == 0) {
        if (n_ok && steps >= 5) tile_of(n_pid, n_first, n_gsz, n_exp, n_mb, n_me, n_nb);
        scale_load(c_mb);
      }
      if (st == 1 && n_ok && steps >= 5) k_of(n_exp, n_kb, n_ks);
      if (st == 2) pf = n_ok && steps >= 5 && n_stages(n_ks) >= NB;
      // this tile's stages, then the next tile's (B from three stages before
      // the end, A from two), or repeats of the last stage
      int sa = st + NA, sb = st + NB;
      if (sb > last) {
        if (pf && sb == last + 1) b_setup(n_exp, n_nb, n_kb);
        sb = pf ? sb - steps : last;
      }
      if (sa > last) {
        if (pf && sa == last + 1) a_offsets(n_kb);
        sa = pf ? sa - steps : last;
      }
      const int live1 = (half_last && st == last) ? 0 : c_live;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int q = 0; q < RD_PER; ++q) {
          const int i = fm * RD_PER + q;
          if (i < NRD) rd(an, bn, 0, i, xa0, xb0);
        }
        if (fm < live1) mrow(fm, xa1, xb1);
#pragma unroll
        for (int q = 0; q < LD_PER; ++q) {
          const int j = fm * LD_PER + q;
          if (j < A_LD) load_a(ac, sa, j);
          else if (j < A_LD + B_LD) load_b(bc, sb, j - A_LD);
        }
        // the next tile's A rows, requested once this tile's last A loads
        // are out (before the stage's B loads, so the next stage's wait
        // covers them) and turned into offsets a stage later
        if (fm == (A_LD - 1) / LD_PER && st == last - NA && pf) a_gather(n_mb, n_me);
        __builtin_amdgcn_sched_barrier(0);
      }
      a_cur = a_nxt;
      b_cur = b_nxt;
    }
    __builtin_amdgcn_s_setprio(0);
    epilogue(c_mb, c_me - c_mb, c_nb, c_exp, c_live);
    if (!n_ok) break;
    if (!pf) {  // (decoded here when the tile was too short to do it on the way)
      group_of(n_pid, n_first, n_gsz);
      tile_of(n_pid, n_first, n_gsz, n_exp, n_mb, n_me, n_nb);
      k_of(n_exp, n_kb, n_ks);
    }
    for (int i = 0; i < FM; ++i)
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    pid = n_pid;
    c_mb = n_mb;
    c_me = n_me;
    c_nb = n_nb;
    c_exp = n_exp;
    c_kb = n_kb;
    c_ks = n_ks;
    primed = pf;
  }
  wait_vm_lgkm0<0>();  // the repeated loads land before the workgroup's LDS is released
}

template <int BM, int BN, int WGM, int WGN, int NA, int EPI, bool BKM = false, bool KS = false>
hipError_t run2(const GemmArgs &a, const GemmArgs *second, hipStream_t s) {
  constexpr int NOUT = EPI == EPI_SWIGLU ? BN / 2 : BN;
  auto bound = [&](GemmArgs &g) {  // m-tile bound (grid size) of one problem
    g.max_mtiles = g.tiles ? g.max_mtiles : (g.M + BM - 1) / BM;
    return g.max_mtiles * ((g.N + NOUT - 1) / NOUT) * (KS && g.k_split > 1 ? g.k_split : 1);
  };
  GemmArgs b0 = a, b1{};
  const int64_t t0 = bound(b0);
  int64_t t1 = 0;
  if (second && second->N > 0) {
    b1 = *second;
    t1 = bound(b1);
  }
  if (t0 + t1 == 0) return hipSuccess;
  const int64_t blocks = 8 * ((t0 + 7) / 8 + (t1 + 7) / 8);  // each problem dealt over 8 XCDs
  gemm2_kernel<BM, BN, WGM, WGN, NA, EPI, BKM, KS>
      <<<static_cast<unsigned>(blocks), 64 * WGM * WGN, 0, s>>>(b0, b1);
  return hipGetLastError();
}

// Compute units of the current device, read once per device.
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 8)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Persistent 256x256 launch: one workgroup per CU (a multiple of 8: whole
// XCDs), none past the tile bound.
template <int EPI>
hipError_t run2p(const GemmArgs &a, hipStream_t s) {
  constexpr int NOUT = EPI == EPI_SWIGLU || EPI == EPI_GLU_F32 ? 128 : 256;
  GemmArgs b = a;
  b.max_mtiles = b.tiles ? b.max_mtiles : (b.M + 255) / 256;
  const int64_t bound = b.max_mtiles * ((b.N + NOUT - 1) / NOUT);
  if (bound == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>(8 * ((bound + 7) / 8), 8 * (cu_count() / 8));
  gemm2p_kernel<EPI><<<static_cast<unsigned>(blocks), 512, 0, s>>>(b);
  return hipGetLastError();
}

// A problem for the persistent form: a register epilogue (K-grouped: the
// fp32 store), a reduction of at least 5 stages (K-grouped: any, a short
// expert's tile starting with a prologue of its own), output rows of at
// most 4 MiB (32-bit store offsets), and at least kMinRounds tiles per
// workgroup (below that the hardware's dynamic dispatch balances better than
// a fixed list).
constexpr int64_t kMinRounds = 2;
bool persistent_one(const GemmArgs &a, int epi) {
  if (a.a2 || a.k_split > 1 || a.b_kmajor) return false;
  if (epi != EPI_SWIGLU && epi != EPI_SCALE && epi != EPI_STORE_F32 && epi != EPI_GLU_F32)
    return false;
  if (a.k_offsets ? epi != EPI_STORE_F32 : (a.K + 63) / 64 < 5) return false;
  if (a.ldo * 4 * 256 >= (int64_t(1) << 32) || (epi == EPI_GLU_F32 && !a.out2)) return false;
  const int64_t mt = a.tiles ? a.max_mtiles : (a.M + 255) / 256;
  const int64_t nout = epi == EPI_SWIGLU || epi == EPI_GLU_F32 ? 128 : 256;
  return mt * ((a.N + nout - 1) / nout) >= kMinRounds * cu_count();
}

template <int BM, int BN, int WGM, int WGN, int NA = 2>
hipError_t dispatch2(const GemmArgs &a, const GemmArgs *b, int epi, hipStream_t s) {
  if (a.k_split > 1 || (b && b->N > 0 && b->k_split > 1)) {  // K split: fp32 store only
    if (epi != EPI_STORE_F32 || a.b_kmajor || (b && b->N > 0 && b->b_kmajor))
      return hipErrorInvalidValue;
    return run2<BM, BN, WGM, WGN, NA, EPI_STORE_F32, false, true>(a, b, s);
  }
  if (a.b_kmajor) {  // K-major B: fp32 store only (backward products)
    if (epi != EPI_STORE_F32 || (b && b->N > 0 && !b->b_kmajor)) return hipErrorInvalidValue;
    return run2<BM, BN, WGM, WGN, NA, EPI_STORE_F32, true>(a, b, s);
  }
  if (b && b->N > 0 && b->b_kmajor) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_SWIGLU: return run2<BM, BN, WGM, WGN, NA, EPI_SWIGLU>(a, b, s);
    case EPI_SCALE: return run2<BM, BN, WGM, WGN, NA, EPI_SCALE>(a, b, s);
    case EPI_STORE: return run2<BM, BN, WGM, WGN, NA, EPI_STORE>(a, b, s);
    case EPI_COMBINE: return run2<BM, BN, WGM, WGN, NA, EPI_COMBINE>(a, b, s);
    case EPI_STORE_F32: return run2<BM, BN, WGM, WGN, NA, EPI_STORE_F32>(a, b, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool gemm2_applicable(const GemmArgs &a, int epi) {
  // K split: fp32 store of one problem, each split whole stages of K and
  // every split holding some
  if (a.k_split > 1) {
    if (epi != EPI_STORE_F32 || a.a2 || a.k_offsets || a.b_kmajor) return false;
    const int64_t stages = (a.K + 63) / 64, kps = (stages + a.k_split - 1) / a.k_split * 64;
    if ((a.k_split - 1) * kps >= a.K) return false;
  }
  // 32-bit load offsets: A (rows it may address), each B slice, below 4 GiB
  // (B offsets run up to one tile past N)
  constexpr int64_t kLim = int64_t(1) << 32;
  const int64_t a_rows = a.a_extent ? a.a_extent : (a.tiles ? 0 : a.M);
  if (a_rows <= 0 || a_rows * a.lda * 2 >= kLim) return false;
  if (a.b_kmajor) {  // [K, N] B: stage offsets run up to 64 rows past K
    if (epi != EPI_STORE_F32 || a.k_offsets || a.ldb % 8 || (a.K + 64LL) * a.ldb * 2 >= kLim)
      return false;
    if (a.a2 && (a.ldb2 % 8 || (a.K2 + 64LL) * a.ldb2 * 2 >= kLim)) return false;
  } else if ((a.N + 256LL) * a.ldb * 2 >= kLim ||
             (a.a2 && (a.N + 256LL) * a.ldb2 * 2 >= kLim)) {
    return false;
  }
  if (a.a2 && a.M * a.lda2 * 2 >= kLim) return false;
  // K a multiple of 32 (64 for the first of two segments)
  if (!a.k_offsets && (a.K % 32 || (a.a2 && (a.K % 64 || a.K2 % 32)))) return false;
  if (a.k_offsets && (!a.tiles || a.a2 || a.a_rows)) return false;
  if (a.N % 8) return false;
  if (epi == EPI_COMBINE && a.ldy % 8) return false;
  return a.ldo % 8 == 0;
}

int gemm2_bm(int cfg) {
  switch (cfg) {
    case TILE2_128x128: case TILE2_128x128_W8D4: return 128;
    case TILE2_64x128: return 64;
    case TILE2_32x256_D2: return 32;
  }
  return 256;
}

int gemm2_bn(int cfg) {
  switch (cfg) {
    case TILE2_128x128: case TILE2_64x128: case TILE2_128x128_W8D4: case TILE2_256x128_W8D3:
      return 128;
  }
  return 256;
}

// Tile of the pipelined kernel for an output of rows x n_out over a reduction
// of K (grouped: `groups` experts, each of which may end in a partial m-tile;
// dense: groups = 0; plus an optional dense rows2 x n_out2 problem sharing the
// launch). From sweeps of every tile on MI355X over the
// benchmark layers: 256x256 wins when it gives each of the 256 CUs two
// workgroups, or one over a long reduction; below that, 128x128 with two
// workgroups per CU (their
// prologues and epilogues overlap the other's K loop), or 256x128 for long
// reductions; with fewer than 256 such tiles, the 8-wavefront 128x128 with a
// deeper look-ahead, and 64x128 for the fewest.
int gemm2_pick(int64_t rows, int64_t groups, int64_t K, int64_t n_out, int glu, int64_t rows2,
               int64_t n_out2) {
  auto tiles = [&](int cfg) {
    const int64_t bm = gemm2_bm(cfg), nout = glu ? gemm2_bn(cfg) / 2 : gemm2_bn(cfg);
    const int64_t mt = groups ? rows / bm + (rows < groups ? rows : groups) : (rows + bm - 1) / bm;
    return mt * ((n_out + nout - 1) / nout) +
           (rows2 > 0 ? ((rows2 + bm - 1) / bm) * ((n_out2 + nout - 1) / nout) : 0);
  };
  constexpr int64_t kCUs = 256;
  const int64_t t256 = tiles(TILE2_256x256_TALLW);
  if (t256 >= 2 * kCUs || (t256 >= kCUs && K >= 1024)) return TILE2_256x256_TALLW;
  if (K >= 2048 && tiles(TILE2_256x128_W8D3) >= kCUs) return TILE2_256x128_W8D3;
  if (tiles(TILE2_128x128) >= kCUs) return TILE2_128x128;
  if (tiles(TILE2_128x128_W8D4) >= kCUs / 2) return TILE2_128x128_W8D4;
  return TILE2_64x128;
}

// Dense GEMM: the pipelined kernel when it applies (bf16, K a multiple of
// 32, more than 64 rows); else the largest generic tile that still gives
// every CU a workgroup (few rows: 16-row tiles, as wide as that allows).
hipError_t launch_dense(const GemmArgs &a, int epi, int act_bf16, hipStream_t s) {
  const int glu = epi == EPI_SWIGLU;
  const int64_t ks = a.k_split > 1 ? a.k_split : 1;
  constexpr int64_t kFill = 256;
  if (a.M <= 64) {
    const bool wide = ks * tile_count(TILE_SMALL_M, a.M, a.N, glu) >= kFill;
    return launch_gemm(a, epi, wide || !act_bf16 ? TILE_SMALL_M : TILE_SMALL_N64, act_bf16, s);
  }
  if (act_bf16 && gemm2_applicable(a, epi))
    return launch_gemm2(a, epi, gemm2_pick(a.M, 0, a.K + (a.a2 ? a.K2 : 0), a.N, glu), s);
  if (!act_bf16) return launch_gemm(a, epi, TILE_LARGE, act_bf16, s);
  for (int cfg : {TILE_LARGE, TILE_TALL_N64, TILE_MID})
    if (ks * tile_count(cfg, a.M, a.N, glu) >= kFill) return launch_gemm(a, epi, cfg, act_bf16, s);
  return launch_gemm(a, epi, TILE_SMALL_N64, act_bf16, s);
}

bool gemm2_persistent(const GemmArgs &a, int epi, int cfg, const GemmArgs *b) {
  return cfg == TILE2_256x256_TALLW && (!b || b->N <= 0) && persistent_one(a, epi);
}

hipError_t launch_gemm2(const GemmArgs &a, int epi, int cfg, hipStream_t s, const GemmArgs *b) {
  switch (cfg) {
    case TILE2_256x256: return dispatch2<256, 256, 2, 4>(a, b, epi, s);
    case TILE2_256x256_TALLW:
      if (gemm2_persistent(a, epi, cfg, b)) {
        switch (epi) {
          case EPI_SWIGLU: return run2p<EPI_SWIGLU>(a, s);
          case EPI_SCALE: return run2p<EPI_SCALE>(a, s);
          case EPI_STORE_F32: return run2p<EPI_STORE_F32>(a, s);
          case EPI_GLU_F32: return run2p<EPI_GLU_F32>(a, s);
        }
      }
      if (epi == EPI_GLU_F32) return hipErrorInvalidValue;  // (persistent kernel only)
      return dispatch2<256, 256, 4, 2>(a, b, epi, s);
    case TILE2_128x128: return dispatch2<128, 128, 2, 2>(a, b, epi, s);
    case TILE2_64x128: return dispatch2<64, 128, 2, 2>(a, b, epi, s);
    case TILE2_128x128_W8D4: return dispatch2<128, 128, 4, 2, 4>(a, b, epi, s);
    case TILE2_256x128_W8D3: return dispatch2<256, 128, 4, 2, 3>(a, b, epi, s);
    case TILE2_32x256_D2: return dispatch2<32, 256, 1, 4, 2>(a, b, epi, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
