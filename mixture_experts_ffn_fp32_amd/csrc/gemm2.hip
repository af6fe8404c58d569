// Pipelined bf16 GEMM for large tiles (gfx950): C = A B^T, same contract and
// epilogues as gemm.hip (grouped expert tiles from a device table or dense;
// row-gathered A; SwiGLU, row-scale, store, fp32 store, combine epilogues;
// optional second K segment).
//
// Main loop. A workgroup of 4 wavefronts owns a BM x BN tile (each
// wavefront a (BM/2) x (BN/2) quarter of 16x16 accumulators on
// v_mfma_f32_16x16x32_bf16). K advances 64 elements (128 bytes per row) per
// stage, two MFMA k-steps. At the start of a stage each thread issues its
// 16-byte global loads of the next stage (8 lanes per 128-byte row
// segment); the stage's MFMAs (2 x 64 per wavefront) then cover their
// latency, and the registers are written to the other LDS buffer before the
// single barrier of the stage. All waits are local to one stage, which the
// compiler's wait-count tracking handles exactly. Within a row the eight
// 16-byte chunks are XOR-swizzled by row & 7 so the 16-byte fragment reads of
// 8 consecutive rows fall in distinct bank groups. (Direct global->LDS
// 16-byte loads were measured to issue per-dword cache accesses on this part
// and are not used.)
//
// K must be a multiple of 64 (every workload's widths are); the host uses
// gemm.hip otherwise. Rows of A past the tile end and columns of B past N
// are read from a valid row (their results are never stored), so loads need
// no predicates.
//
// Epilogue. Each wavefront stages its accumulators through LDS 16 rows at a
// time and writes the output with 16-byte stores along rows; the combine
// epilogue adds the token's K routed rows with 16-byte loads.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#ifndef MOE_G2_PIPE
#define MOE_G2_PIPE 1
#endif
#ifndef MOE_G2_ROLL
#define MOE_G2_ROLL 1
#endif
#ifndef MOE_G2_DMA
#define MOE_G2_DMA 1
#endif

constexpr int kMaxStageBytes = (256 + 256) * 128;  // largest tile, one stage
// direct-to-LDS loads: two A buffers and three B buffers of one stage each
constexpr int kLdsBytes = MOE_G2_DMA ? (2 * 256 + 3 * 256) * 128 : 2 * kMaxStageBytes;

// stage buffers, back to back
__shared__ __attribute__((aligned(1024))) u32x4 g2_lds[kLdsBytes / 16];
#define g2_s0 (g2_lds)
#define g2_s1 (g2_lds + kMaxStageBytes / 16)

// s_waitcnt with vmcnt = n (<= 63), lgkmcnt = 0, expcnt untouched.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// 16-byte direct-to-LDS load: lane i's data lands at lds + 16 i (lds is
// wave-uniform). (Device-pass only: the host pass does not know the builtin.)
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, u32x4 *lds, uint32_t voff,
                                           int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                           voff, soff, 0, 0);
#endif
}

__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// physical 16-byte chunk of logical chunk c in row r (rows of 8 chunks)
__device__ __forceinline__ int sw8(int r, int c) { return r * 8 + (c ^ (r & 7)); }

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + __expf(-x)); }


template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256, 1) void gemm2_kernel(GemmArgs p) {
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr bool GLU = EPI == EPI_SWIGLU;
  constexpr int NOUT = GLU ? BN / 2 : BN;
  constexpr int A_LD = BM / 32, B_LD = BN / 32;  // 16-byte loads per thread per stage
  constexpr int STAGE16 = (BM + BN) * 8;        // 16-byte units per stage
  static_assert(STAGE16 * 16 <= kMaxStageBytes, "stage fits");
  static_assert(!GLU || FN % 2 == 0, "paired gate/up fragments");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ------------------------------------------------------------ tile
  const int n_tn = (p.N + NOUT - 1) / NOUT;
  const int64_t n_m = p.tiles ? static_cast<int64_t>(*p.n_tiles) : p.max_mtiles;
  const int64_t total = n_m * n_tn;
  const int64_t per = (total + 7) / 8;
  const int64_t local = blockIdx.x >> 3;
  if (local >= per) return;
  const int64_t pid = static_cast<int64_t>(blockIdx.x & 7) * per + local;
  if (pid >= total) return;
  constexpr int GM = 4;
  const int64_t grp = pid / (GM * n_tn);
  const int64_t first_m = grp * GM;
  const int gsz = static_cast<int>(min<int64_t>(n_m - first_m, GM));
  const int64_t in_g = pid - grp * GM * n_tn;
  const int64_t mt = first_m + in_g % gsz;
  const int nt = static_cast<int>(in_g / gsz);
  int64_t expert = 0, m_begin, m_end;
  if (p.tiles) {
    expert = __builtin_amdgcn_readfirstlane(p.tiles[3 * mt]);
    m_begin = __builtin_amdgcn_readfirstlane(p.tiles[3 * mt + 1]);
    m_end = __builtin_amdgcn_readfirstlane(p.tiles[3 * mt + 2]);
  } else {
    m_begin = mt * BM;
    m_end = min<int64_t>(m_begin + BM, p.M);
  }
  const int n_begin = nt * NOUT;

  // ------------------------------------------------------------ loaders
  // load j of a thread covers tile row (tid / 8 + 32 j), logical chunk tid % 8
  const int lrow = tid >> 3;
  const int lchunk = tid & 7;
  // chunk this thread fetches: its own (registers, swizzled on the LDS
  // write), or the one its LDS slot holds (direct-to-LDS loads land at
  // lane-consecutive addresses)
  const int lchunk_g = MOE_G2_DMA ? (lchunk ^ (lrow & 7)) : lchunk;
  // Loads go through buffer resources: a uniform base and byte extent per
  // operand (per gate / up half, per expert) and a 32-bit offset per load
  // (extents below 4 GiB are a launch precondition); the stage's k offset is
  // the scalar offset. Accesses past an extent would read zeros.
  auto rsrc = [](const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0,
                                             static_cast<int>(static_cast<uint32_t>(bytes)),
                                             0x00020000);
  };
  __amdgpu_buffer_rsrc_t ar, br0, br1;
  uint32_t aoff[A_LD];
  uint32_t boff0 = 0, bstep = 0;  // B: row lrow's offset; 32 rows further (uniform)
  // operand set-up for K segment seg (A and B separately: the direct-to-LDS
  // pipeline requests B a stage further ahead than A)
  auto setup_a = [&](int seg) {
    if (seg && !p.a2) return;  // no second K segment: keep the first segment's rows
    const int64_t lda = seg ? p.lda2 : p.lda;
    const int64_t a_rows = seg ? p.M : (p.a_extent ? p.a_extent : p.M);
    ar = rsrc(seg ? p.a2 : p.a, a_rows * lda * 2);
#pragma unroll
    for (int j = 0; j < A_LD; ++j) {
      const int r = lrow + 32 * j;
      int64_t m = m_begin + r;
      if (m >= m_end) m = m_begin;  // results of these rows are never stored
      const int64_t src = (!seg && p.a_rows) ? static_cast<int64_t>(p.a_rows[m]) : m;
      aoff[j] = static_cast<uint32_t>((src * lda + lchunk_g * 8) * 2);
    }
  };
  auto setup_b = [&](int seg) {
    if (seg && !p.a2) return;
    // B rows past N lie past the resource's extent and read as zeros
    const int64_t ldb = seg ? p.ldb2 : p.ldb, bytes = static_cast<int64_t>(p.N) * ldb * 2;
    if (seg) {
      br0 = br1 = rsrc(p.b2, bytes);
    } else {
      const int64_t eoff = expert * p.b_stride * 2;
      br0 = rsrc(static_cast<const char *>(p.b0) + eoff, bytes);
      br1 = GLU ? rsrc(static_cast<const char *>(p.b1) + eoff, bytes) : br0;
    }
    boff0 = static_cast<uint32_t>((static_cast<int64_t>(n_begin + lrow) * ldb + lchunk_g * 8) * 2);
    bstep = static_cast<uint32_t>(32 * ldb * 2);
  };
  auto setup = [&](int seg) {
    setup_a(seg);
    setup_b(seg);
  };

  const int steps1 = p.K / 64;
  const int steps = steps1 + (p.a2 ? p.K2 / 64 : 0);

  // registers of the next stage
  u32x4 ra[A_LD], rb[B_LD];
  auto load_one = [&](int st, int j) {
    const int kb = __builtin_amdgcn_readfirstlane((st >= steps1 ? st - steps1 : st) * 128);
    if (j < A_LD) {
      ra[j] = __builtin_amdgcn_raw_buffer_load_b128(ar, aoff[j], kb, 0);
    } else {
      const int jb = j - A_LD;  // gate rows first, then up rows (SwiGLU)
      const bool up = GLU && jb >= B_LD / 2;
      rb[jb] = __builtin_amdgcn_raw_buffer_load_b128(
          up ? br1 : br0, boff0 + (up ? jb - B_LD / 2 : jb) * bstep, kb, 0);
    }
  };
  auto load = [&](int st) {
#pragma unroll
    for (int j = 0; j < A_LD + B_LD; ++j) load_one(st, j);
  };
  auto put = [&](u32x4 *buf) {
#pragma unroll
    for (int j = 0; j < A_LD; ++j) buf[sw8(lrow + 32 * j, lchunk)] = ra[j];
#pragma unroll
    for (int j = 0; j < B_LD; ++j) buf[BM * 8 + sw8(lrow + 32 * j, lchunk)] = rb[j];
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment rows: A row of fm, B row of fn (within the stage)
  const int fr = lane & 15, fc = lane >> 4;
  auto brow_of = [&](int fn) {
    if (GLU) {
      constexpr int half = FN / 2;
      return fn < half ? wn * (WTN / 2) + fn * 16 : BN / 2 + wn * (WTN / 2) + (fn - half) * 16;
    }
    return wn * WTN + fn * 16;
  };
  // number of this wave's 16-row fragments that hold rows of the tile
  const int64_t rows_left = m_end - (m_begin + wm * WTM);
  const int fm_live = rows_left <= 0 ? 0 : (rows_left >= WTM ? FM : static_cast<int>((rows_left + 15) / 16));

  const int live = __builtin_amdgcn_readfirstlane(fm_live);
#if MOE_G2_DMA
  // Direct-to-LDS pipeline. Each 16-byte load of a thread lands in LDS at
  // its lane's slot of a 1 KB block (8 rows of 128 bytes), so the thread
  // fetches the logical chunk that slot holds under the row swizzle. A has
  // two stage buffers and B three, so B (the streamed weights) is requested
  // two stages ahead and A one. Per stage s (A buffer s % 2, B buffer s % 3):
  //   M0: MFMAs of k-step 0 (fragment set 0), interleaved with the reads of
  //       k-step 1 (set 1) from the stage's buffers;
  //   wait until A and B of stage s + 1 have landed (B of s + 2 may still
  //       be in flight), lgkmcnt 0, barrier: stage s + 1 is visible and
  //       stage s's buffers are free;
  //   M1: MFMAs of set 1, interleaved with the loads of A(s + 2) and
  //       B(s + 3) into the freed buffers and the reads of k-step 0 of
  //       stage s + 1 (set 0).
  // Loads past the last stage repeat it (their buffers are never read).
  constexpr int A16 = BM * 8, B16 = BN * 8;  // 16-byte units per stage buffer
  u32x4 *const abuf = g2_lds;                // A: 2 x A16
  u32x4 *const bbuf = g2_lds + 2 * A16;      // B: 3 x B16
  static_assert((2 * A16 + 3 * B16) * 16 <= kLdsBytes, "stage buffers fit");
  bf16x8 xa0[FM], xb0[FN], xa1[FM], xb1[FN];
  auto rd = [&](const u32x4 *ab, const u32x4 *bb, int ks, int i, bf16x8 *xa, bf16x8 *xb) {
    const int kc = 4 * ks + fc;
    if (i < FN)
      xb[i] = __builtin_bit_cast(bf16x8, bb[sw8(brow_of(i) + fr, kc)]);
    else
      xa[i - FN] = __builtin_bit_cast(bf16x8, ab[sw8(wm * WTM + (i - FN) * 16 + fr, kc)]);
  };
  auto mrow = [&](int fm, const bf16x8 *xa, const bf16x8 *xb) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
      acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[fm], xb[fn], acc[fm][fn], 0, 0, 0);
  };
  // load j of a stage: rows 32 j + lrow; the wave's 1 KB block starts at
  // row 32 j + 8 wave
  auto dma_a = [&](u32x4 *ab, int st, int j) {
    const int kb = __builtin_amdgcn_readfirstlane((st >= steps1 ? st - steps1 : st) * 128);
    load_lds16(ar, ab + (32 * j + 8 * wave) * 8, aoff[j], kb);
  };
  auto dma_b = [&](u32x4 *bb, int st, int j) {
    const int kb = __builtin_amdgcn_readfirstlane((st >= steps1 ? st - steps1 : st) * 128);
    const bool up = GLU && j >= B_LD / 2;
    load_lds16(up ? br1 : br0, bb + (32 * j + 8 * wave) * 8, boff0 + (up ? j - B_LD / 2 : j) * bstep,
               kb);
  };
  constexpr int NRD = FM + FN;
  constexpr int RD_PER = (NRD + FM - 1) / FM;
  constexpr int LD_PER = (A_LD + B_LD + FM - 1) / FM;

  // (stages are requested in order per operand; an operand switches to the
  // second K segment's rows before its first load from that segment)
  setup(0);
  const int last = steps - 1;
  auto seg_a = [&](int st) {
    if (st == steps1) setup_a(1);
  };
  auto seg_b = [&](int st) {
    if (st == steps1) setup_b(1);
  };
#pragma unroll
  for (int j = 0; j < A_LD; ++j) dma_a(abuf, 0, j);
#pragma unroll
  for (int j = 0; j < B_LD; ++j) dma_b(bbuf, 0, j);
  seg_a(min(1, last));
  seg_b(min(1, last));
#pragma unroll
  for (int j = 0; j < A_LD; ++j) dma_a(abuf + A16, min(1, last), j);
#pragma unroll
  for (int j = 0; j < B_LD; ++j) dma_b(bbuf + B16, min(1, last), j);
  seg_b(min(2, last));
#pragma unroll
  for (int j = 0; j < B_LD; ++j) dma_b(bbuf + 2 * B16, min(2, last), j);
  wait_vm_lgkm0<2 * B_LD + A_LD>();  // stage 0 has landed
  barrier();
#pragma unroll
  for (int i = 0; i < NRD; ++i) rd(abuf, bbuf, 0, i, xa0, xb0);

  int b_cur = 0;  // s % 3
  for (int st = 0; st < steps; ++st) {
    const int a_cur = st & 1;
    const int b_nxt = b_cur == 2 ? 0 : b_cur + 1;
    u32x4 *const ac = abuf + a_cur * A16, *const an = abuf + (a_cur ^ 1) * A16;
    u32x4 *const bc = bbuf + b_cur * B16, *const bn = bbuf + b_nxt * B16;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): set 0 has landed
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if (fm < live) mrow(fm, xa0, xb0);
#pragma unroll
      for (int q = 0; q < RD_PER; ++q) {
        const int i = fm * RD_PER + q;
        if (i < NRD) rd(ac, bc, 1, i, xa1, xb1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vm_lgkm0<B_LD>();  // A and B of st + 1 have landed
    barrier();
    const int sa = min(st + 2, last), sb = min(st + 3, last);
    if (st + 2 <= last) seg_a(sa);
    if (st + 3 <= last) seg_b(sb);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if (fm < live) mrow(fm, xa1, xb1);
#pragma unroll
      for (int q = 0; q < LD_PER; ++q) {
        const int j = fm * LD_PER + q;
        if (j < A_LD) dma_a(ac, sa, j);
        else if (j < A_LD + B_LD) dma_b(bc, sb, j - A_LD);
      }
#pragma unroll
      for (int q = 0; q < RD_PER; ++q) {
        const int i = fm * RD_PER + q;
        if (i < NRD) rd(an, bn, 0, i, xa0, xb0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    b_cur = b_nxt;
  }
  wait_vm_lgkm0<0>();
  barrier();  // the epilogue reuses the stage buffers
#elif MOE_G2_PIPE
  // Software pipeline over half-stages (one MFMA k-step each). Fragment
  // registers come in two sets: set 0 holds k-step 0 of the current stage,
  // set 1 k-step 1. Per stage, with `cur` the stage's LDS buffer:
  //   M0: MFMAs of set 0, interleaved row by row with the reads of set 1
  //       (from cur), the LDS writes of the next stage into the other buffer
  //       (from the staging registers) and the global loads of the stage
  //       after next into the freed staging registers;
  //   barrier (after lgkmcnt 0): the next stage is visible, and every read
  //       of the other buffer issued before it has completed;
  //   M1: MFMAs of set 1, interleaved with the reads of the next stage's
  //       k-step 0 into set 0.
  // Each MFMA group's operands were requested one half-stage earlier, and the
  // global loads have a full stage to land. sched_barrier keeps this order.
  bf16x8 xa0[FM], xb0[FN], xa1[FM], xb1[FN];
  auto rd = [&](const u32x4 *buf, int ks, int i, bf16x8 *xa, bf16x8 *xb) {
    const int kc = 4 * ks + fc;
    if (i < FN)
      xb[i] = __builtin_bit_cast(bf16x8, buf[BM * 8 + sw8(brow_of(i) + fr, kc)]);
    else
      xa[i - FN] = __builtin_bit_cast(bf16x8, buf[sw8(wm * WTM + (i - FN) * 16 + fr, kc)]);
  };
  auto mrow = [&](int fm, const bf16x8 *xa, const bf16x8 *xb) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
      acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[fm], xb[fn], acc[fm][fn], 0, 0, 0);
  };
  constexpr int NRD = FM + FN;              // fragment reads per set
  constexpr int RD_PER = (NRD + FM - 1) / FM;
  constexpr int WR_PER = (A_LD + B_LD + FM - 1) / FM;
  auto put_one = [&](u32x4 *buf, int j) {
    if (j < A_LD) buf[sw8(lrow + 32 * j, lchunk)] = ra[j];
    else buf[BM * 8 + sw8(lrow + 32 * (j - A_LD), lchunk)] = rb[j - A_LD];
  };

  setup(0);
  load(0);
  put(g2_s0);
  if (steps1 == 1 && steps > 1) setup(1);
  load(steps > 1 ? 1 : 0);
  barrier();
#pragma unroll
  for (int i = 0; i < NRD; ++i) rd(g2_s0, 0, i, xa0, xb0);
  // One stage from CUR; NXT receives the next stage. Near the end the loads
  // repeat the last stage and the next-stage writes and reads are unused,
  // so the body has no conditions beyond the rows check of partial tiles.
#define G2_STAGE(ST, CUR, NXT)                                                   \
  {                                                                              \
    const int st_ = (ST);                                                        \
    if (st_ >= steps) break;                                                     \
    if (st_ + 2 == steps1 && st_ + 2 < steps) setup(1);                          \
    const int ld_ = st_ + 2 < steps ? st_ + 2 : steps - 1;                       \
    __builtin_amdgcn_s_waitcnt(0xC07F); /* lgkmcnt(0): set 0 has landed */       \
    _Pragma("unroll") for (int fm = 0; fm < FM; ++fm) {                          \
      if (fm < live) mrow(fm, xa0, xb0);                                         \
      _Pragma("unroll") for (int q = 0; q < RD_PER; ++q) {                       \
        const int i = fm * RD_PER + q;                                           \
        if (i < NRD) rd(CUR, 1, i, xa1, xb1);                                    \
      }                                                                          \
      _Pragma("unroll") for (int q = 0; q < WR_PER; ++q) {                       \
        const int j = fm * WR_PER + q;                                           \
        if (j < A_LD + B_LD) {                                                   \
          put_one(NXT, j);                                                       \
          load_one(ld_, j);                                                      \
        }                                                                        \
      }                                                                          \
      __builtin_amdgcn_sched_barrier(0);                                         \
    }                                                                            \
    __builtin_amdgcn_s_waitcnt(0xC07F); /* lgkmcnt(0) */                         \
    barrier();                                                                   \
    _Pragma("unroll") for (int fm = 0; fm < FM; ++fm) {                          \
      if (fm < live) mrow(fm, xa1, xb1);                                         \
      _Pragma("unroll") for (int q = 0; q < RD_PER; ++q) {                       \
        const int i = fm * RD_PER + q;                                           \
        if (i < NRD) rd(NXT, 0, i, xa0, xb0);                                    \
      }                                                                          \
      __builtin_amdgcn_sched_barrier(0);                                         \
    }                                                                            \
  }
#if MOE_G2_ROLL
  // one stage per iteration, buffers picked by parity (one register
  // assignment for the loop-carried fragments and staging registers)
  for (int st = 0; st < steps; ++st) {
    u32x4 *cur = g2_lds + (st & 1) * (kMaxStageBytes / 16);
    u32x4 *nxt = g2_lds + ((st & 1) ^ 1) * (kMaxStageBytes / 16);
    G2_STAGE(st, cur, nxt)
  }
#else
  for (int st = 0; st < steps; st += 2) {
    G2_STAGE(st + 0, g2_s0, g2_s1)
    G2_STAGE(st + 1, g2_s1, g2_s0)
  }
#endif
#undef G2_STAGE
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  barrier();  // the epilogue reuses the stage buffers
#else
  // all fragments are read first (rows past the tile read stale LDS, and
  // their MFMAs are skipped), so the MFMAs issue back to back
  auto compute = [&](const u32x4 *buf) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kc = 4 * ks + fc;
      bf16x8 bf[FN], af[FM];
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        bf[fn] = __builtin_bit_cast(bf16x8, buf[BM * 8 + sw8(brow_of(fn) + fr, kc)]);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        af[fm] = __builtin_bit_cast(bf16x8, buf[sw8(wm * WTM + fm * 16 + fr, kc)]);
      // keep the reads ahead of the branches below (then MFMAs back to back)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) asm volatile("" : "+v"(af[fm]));
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        if (fm < live) {
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            acc[fm][fn] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm], bf[fn], acc[fm][fn], 0, 0, 0);
        }
      }
    }
  };

  setup(0);
  load(0);
  put(g2_s0);
  barrier();
  // Step st: issue the loads of stage st + 1, run the MFMAs of stage st from
  // LDS buffer st % 2, write stage st + 1 into the other buffer, barrier.
  // Unrolled by two so the buffers are named statically.
#define G2_STAGE(ST, CUR, NXT)                  \
  {                                             \
    const int st_ = (ST);                       \
    if (st_ >= steps) break;                    \
    const bool more_ = st_ + 1 < steps;         \
    if (more_) {                                \
      if (st_ + 1 == steps1) setup(1);          \
      load(st_ + 1);                            \
    }                                           \
    compute(CUR);                               \
    if (more_) put(NXT);                        \
    barrier();                                  \
  }
  for (int st = 0; st < steps; st += 2) {
    G2_STAGE(st + 0, g2_s0, g2_s1)
    G2_STAGE(st + 1, g2_s1, g2_s0)
  }
#undef G2_STAGE
#endif

  // ------------------------------------------------------------ epilogue
  // each wave: 16 rows x (OUT cols) of fp32 at a time in its 8 KB+ slice
  constexpr int OUTW = GLU ? WTN / 2 : WTN;   // output columns per wave
  constexpr int FO = GLU ? FN / 2 : FN;
  constexpr int PITCH = OUTW + 4;             // floats per staged row
  float *stg = reinterpret_cast<float *>(wave < 2 ? g2_s0 : g2_s1) + (wave & 1) * 16 * PITCH;
  static_assert(2 * 16 * PITCH * 4 <= kMaxStageBytes, "epilogue staging fits");
  const int col0 = n_begin + (GLU ? wn * (WTN / 2) : wn * WTN);
  constexpr int ITEMS = 16 * OUTW / 8;        // (row, 8-column) items per 16 rows
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    if (fm >= live) break;  // unrolled: acc is indexed statically and stays in registers
#pragma unroll
    for (int fo = 0; fo < FO; ++fo)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = acc[fm][fo][i];
        if (GLU) v = silu_f(v) * acc[fm][fo + FO][i];
        stg[(4 * fc + i) * PITCH + fo * 16 + fr] = v;
      }
    __builtin_amdgcn_s_waitcnt(0xC07F & ~0x0F00);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int it = 0; it < (ITEMS + 63) / 64; ++it) {
      const int item = it * 64 + lane;
      if (item >= ITEMS) break;
      const int r = item / (OUTW / 8), c8 = (item % (OUTW / 8)) * 8;
      const int64_t m = m_begin + wm * WTM + fm * 16 + r;
      const int col = col0 + c8;
      if (m >= m_end || col >= p.N) continue;
      float v[8];
      const float4 lo = *reinterpret_cast<const float4 *>(stg + r * PITCH + c8);
      const float4 hi = *reinterpret_cast<const float4 *>(stg + r * PITCH + c8 + 4);
      v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
      v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
      if (EPI == EPI_SCALE && p.row_scale) {
        const float s = p.row_scale[m];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] *= s;
      }
      if (EPI == EPI_COMBINE) {
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
        for (int e = 0; e < 8; ++e) v[e] += rs[e];
      }
      if (EPI == EPI_STORE_F32) {
        float *o = static_cast<float *>(p.out) + m * p.ldo + col;
        *reinterpret_cast<float4 *>(o) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4 *>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
      } else {
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p.out) + m * p.ldo + col) =
            Chunk<bf16_t>::pack(v);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F & ~0x0F00);  // lgkmcnt(0): reads done before rewrite
    asm volatile("" ::: "memory");
  }
}

template <int BM, int BN, int EPI>
hipError_t run2(const GemmArgs &a, hipStream_t s) {
  constexpr int NOUT = EPI == EPI_SWIGLU ? BN / 2 : BN;
  const int64_t n_tn = (a.N + NOUT - 1) / NOUT;
  const int64_t max_m = a.tiles ? a.max_mtiles : (a.M + BM - 1) / BM;
  const int64_t total = max_m * n_tn;
  if (total == 0) return hipSuccess;
  GemmArgs b = a;
  b.max_mtiles = max_m;
  const int64_t blocks = 8 * ((total + 7) / 8);
  gemm2_kernel<BM, BN, EPI><<<static_cast<unsigned>(blocks), 256, 0, s>>>(b);
  return hipGetLastError();
}

template <int BM, int BN>
hipError_t dispatch2(const GemmArgs &a, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_SWIGLU: return run2<BM, BN, EPI_SWIGLU>(a, s);
    case EPI_SCALE: return run2<BM, BN, EPI_SCALE>(a, s);
    case EPI_STORE: return run2<BM, BN, EPI_STORE>(a, s);
    case EPI_COMBINE: return run2<BM, BN, EPI_COMBINE>(a, s);
    case EPI_STORE_F32: return run2<BM, BN, EPI_STORE_F32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool gemm2_applicable(const GemmArgs &a, int epi) {
  if (a.k_split > 1) return false;
  // 32-bit load offsets: A (rows it may address), each B slice, below 4 GiB
  // (B offsets run up to one tile past N)
  constexpr int64_t kLim = int64_t(1) << 32;
  const int64_t a_rows = a.a_extent ? a.a_extent : (a.tiles ? 0 : a.M);
  if (a_rows <= 0 || a_rows * a.lda * 2 >= kLim || (a.N + 256LL) * a.ldb * 2 >= kLim)
    return false;
  if (a.a2 && (a.M * a.lda2 * 2 >= kLim || (a.N + 256LL) * a.ldb2 * 2 >= kLim)) return false;
  if (a.K % 64 || (a.a2 && a.K2 % 64)) return false;
  if (a.N % 8) return false;
  if (epi == EPI_COMBINE && a.ldy % 8) return false;
  return a.ldo % 8 == 0;
}

int gemm2_bm(int cfg) { return cfg == TILE2_128x256 ? 128 : 256; }

#ifndef MOE_V2_MIN_TILES
#define MOE_V2_MIN_TILES 200
#endif

int64_t gemm2_min_tiles() { return MOE_V2_MIN_TILES; }

// Dense GEMM: the pipelined kernel when it applies and its tile count fills
// the chip; else the largest generic tile that still gives every CU a
// workgroup (few rows: 16-row tiles, as wide as that allows).
hipError_t launch_dense(const GemmArgs &a, int epi, int act_bf16, hipStream_t s) {
  const int glu = epi == EPI_SWIGLU;
  const int64_t ks = a.k_split > 1 ? a.k_split : 1;
  constexpr int64_t kFill = 256;
  if (a.M <= 64) {
    const bool wide = ks * tile_count(TILE_SMALL_M, a.M, a.N, glu) >= kFill;
    return launch_gemm(a, epi, wide || !act_bf16 ? TILE_SMALL_M : TILE_SMALL_N64, act_bf16, s);
  }
  if (act_bf16 && gemm2_applicable(a, epi)) {
    const int64_t nout = glu ? 128 : 256;
    const int64_t tiles = ((a.M + 255) / 256) * ((a.N + nout - 1) / nout);
    if (tiles >= MOE_V2_MIN_TILES) return launch_gemm2(a, epi, TILE2_256x256, s);
  }
  if (!act_bf16) return launch_gemm(a, epi, TILE_LARGE, act_bf16, s);
  for (int cfg : {TILE_LARGE, TILE_TALL_N64, TILE_MID})
    if (ks * tile_count(cfg, a.M, a.N, glu) >= kFill) return launch_gemm(a, epi, cfg, act_bf16, s);
  return launch_gemm(a, epi, TILE_SMALL_N64, act_bf16, s);
}

hipError_t launch_gemm2(const GemmArgs &a, int epi, int cfg, hipStream_t s) {
  switch (cfg) {
    case TILE2_256x256: return dispatch2<256, 256>(a, epi, s);
    case TILE2_256x128: return dispatch2<256, 128>(a, epi, s);
    case TILE2_128x256: return dispatch2<128, 256>(a, epi, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
