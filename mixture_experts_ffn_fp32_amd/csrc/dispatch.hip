// Sorted dispatch of the T*K (token, slot) assignments by expert id.
//
// "StableLatentMoE and QuantileBalancer", section "Dispatch is a stable
// permutation, not token duplication in model state": the flattened expert
// ids are sorted stably, sorted_token = order / K, counts by bincount and
// cumulative ends mark each expert's slice. Here the sort is a counting
// sort, with no host round trip: for up to 16384 slots and 256 experts one
// workgroup does it all (dispatch_fused_kernel); otherwise three launches:
//   hist    - per chunk of 4096 slots, an LDS histogram of expert ids;
//   scan    - one workgroup: counts, exclusive offsets, the absolute base of
//             every (chunk, expert) pair, the grouped-GEMM m-tile table and
//             the near-tie count of the router gaps (below 2^21 slots with
//             one packed 64-bit scan: scan_packed_kernel);
//   scatter - per chunk, rank of each slot among earlier slots of the same
//             expert (64-lane peer masks from one ballot per id bit, waves
//             of the workgroup taking turns on an LDS running count), then
//             perm / sorted_token / inv / sorted_w writes.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kMaxE = 1024;
constexpr int kFusedMaxE = 256;  // experts of the one-workgroup dispatch

__global__ __launch_bounds__(256) void hist_kernel(const int32_t *__restrict__ idx, int64_t slots,
                                                   int E, int32_t *__restrict__ chunk_hist) {
  __shared__ int h[kMaxE];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t s0 = static_cast<int64_t>(blockIdx.x) * kChunkSlots;
  const int64_t s1 = min<int64_t>(s0 + kChunkSlots, slots);
  constexpr int kRounds = kChunkSlots / 256;
  int ids[kRounds];  // all of the chunk's ids requested before the first atomic
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int64_t s = s0 + 256 * r + threadIdx.x;
    ids[r] = s < s1 ? idx[s] : -1;
  }
#pragma unroll
  for (int r = 0; r < kRounds; ++r)
    if (ids[r] >= 0 && ids[r] < E) atomicAdd(&h[ids[r]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    chunk_hist[static_cast<int64_t>(blockIdx.x) * E + e] = h[e];
}

#ifndef MOE_TILE_EVEN
#define MOE_TILE_EVEN 1
#endif
// Rows [begin, end) of m-tile j of n over an expert's R rows starting at
// row0: n = ceil(R / bm) tiles of R / n rows each (the first R % n one row
// more), so an expert just past a multiple of bm rows does not end in a
// tile of a few rows that costs nearly a full one.
__device__ __forceinline__ void tile_rows(int row0, int R, int n, int j, int bm, int *begin,
                                          int *end) {
  if (MOE_TILE_EVEN) {
    *begin = row0 + static_cast<int>(static_cast<int64_t>(j) * R / n);
    *end = row0 + static_cast<int>(static_cast<int64_t>(j + 1) * R / n);
  } else {
    *begin = row0 + j * bm;
    *end = min(*begin + bm, row0 + R);
  }
}

// m-tile tables of height at most bm from offsets held in LDS (1024
// threads), in two steps so that callers can put every global write after
// their last barrier: tile_starts (LDS only: start[e] = first tile of expert
// e, start[E] = total) and write_tiles (global writes only). Tile i =
// {expert, row_begin, row_end, group_first, group_size}; experts with no rows
// get no tile. A group is a run of at most kTileGroup m-tiles of one expert
// (the GEMMs schedule a group's tiles together so they share the expert's
// weight slices in L2).
__device__ void tile_starts(const int *off, int E, int bm, int *start, int *tmp) {
  const int t = threadIdx.x;
  int nt = 0;
  if (t < E) nt = (off[t + 1] - off[t] + bm - 1) / bm;
  int total;
  const int ex = block_exscan_1024(nt, tmp, &total);
  if (t < E) start[t] = ex;
  if (t == 0) start[E] = total;
}

__device__ void write_tiles(const int *off, int E, int bm, const int *start, int32_t *tiles,
                            int32_t *n_tiles) {
  const int t = threadIdx.x;
  const int total = start[E];
  for (int i = t; i < total; i += 1024) {
    int lo = 0, hi = E;  // find e with start[e] <= i < start[e+1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (start[mid] <= i) lo = mid; else hi = mid;
    }
    const int e = lo;
    int r0, r1;
    tile_rows(off[e], off[e + 1] - off[e], start[e + 1] - start[e], i - start[e], bm, &r0, &r1);
    const int gfirst = start[e] + (i - start[e]) / kTileGroup * kTileGroup;
    int32_t *ti = tiles + kTileInts * static_cast<int64_t>(i);
    ti[0] = e;
    ti[1] = r0;
    ti[2] = r1;
    ti[3] = gfirst;
    ti[4] = min(kTileGroup, start[e + 1] - gfirst);
  }
  if (t == 0) *n_tiles = total;
}

__device__ void build_tiles(const int *off, int E, int bm, int *start, int *tmp,
                            int32_t *tiles, int32_t *n_tiles) {
  tile_starts(off, E, bm, start, tmp);
  __syncthreads();
  write_tiles(off, E, bm, start, tiles, n_tiles);
}

__global__ __launch_bounds__(1024) void scan_kernel(ScanArgs a) {
  __shared__ int tmp[1024];
  __shared__ int off[kMaxE + 1];
  __shared__ int start[kMaxE + 1];
  const int t = threadIdx.x;
  const int64_t nch = n_chunks(a.slots);
  // per expert: total over chunks, then each chunk's absolute base; the
  // chunk counts are read kBatch at a time so their loads overlap (chunk_base
  // may alias chunk_hist: each element is read before it is written)
  constexpr int kBatch = 16;
  int cnt = 0;
  if (t < a.E) {
    for (int64_t c0 = 0; c0 < nch; c0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        v[j] = c0 + j < nch ? a.chunk_hist[(c0 + j) * a.E + t] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) cnt += v[j];
    }
  }
  int total;
  const int ex = block_exscan_1024(t < a.E ? cnt : 0, tmp, &total);
  if (t < a.E) {
    off[t] = ex;
    a.counts[t] = cnt;
    a.offsets[t] = ex;
    int run = ex;
    for (int64_t c0 = 0; c0 < nch; c0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        v[j] = c0 + j < nch ? a.chunk_hist[(c0 + j) * a.E + t] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (c0 + j < nch) {
          a.chunk_base[(c0 + j) * a.E + t] = run;
          run += v[j];
        }
    }
  }
  if (t == 0) {
    off[a.E] = total;
    a.offsets[a.E] = total;
  }
  __syncthreads();
  if (a.tiles) build_tiles(off, a.E, a.bm, start, tmp, a.tiles, a.n_tiles);
  __syncthreads();
  if (a.tiles2) build_tiles(off, a.E, a.bm2, start, tmp, a.tiles2, a.n_tiles2);
  __syncthreads();
  if (a.gap && a.n_near_ties) {
    int n = 0;
    for (int64_t i0 = t; i0 < a.T; i0 += 1024 * kBatch) {
      float gv[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int64_t i = i0 + 1024 * j;
        gv[j] = i < a.T ? a.gap[i] : INFINITY;
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) n += (gv[j] < a.tie_eps) ? 1 : 0;
    }
    int tot;
    block_exscan_1024(n, tmp, &tot);
    if (t == 0) *a.n_near_ties = tot;
  }
}

__global__ __launch_bounds__(1024) void tiles_kernel(const int32_t *offsets, int E, int bm,
                                                     int32_t *tiles, int32_t *n_tiles) {
  __shared__ int tmp[1024];
  __shared__ int off[kMaxE + 1];
  __shared__ int start[kMaxE + 1];
  for (int e = threadIdx.x; e <= E; e += 1024) off[e] = offsets[e];
  __syncthreads();
  build_tiles(off, E, bm, start, tmp, tiles, n_tiles);
}

__global__ __launch_bounds__(256) void scatter_kernel(ScatterArgs a) {
  __shared__ int run[kMaxE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int e = tid; e < a.E; e += 256) run[e] = 0;
  __syncthreads();
  int bits = 0;
  while ((1 << bits) < a.E) ++bits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t c = blockIdx.x;
  const int64_t s0 = c * kChunkSlots;
  const int64_t s1 = min<int64_t>(s0 + kChunkSlots, a.slots);
  const int32_t *base = a.chunk_base + c * a.E;
  constexpr int kRounds = kChunkSlots / 256;
  int ids[kRounds];  // the chunk's ids and weights, all requested up front
  float gs[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int64_t s = s0 + 256 * r + tid;
    ids[r] = s < s1 ? a.idx[s] : -1;
    gs[r] = (s < s1 && a.sorted_w) ? a.g[s] : 0.f;
  }
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int64_t s = s0 + 256 * r + tid;
    const int e = ids[r];
    const bool valid = e >= 0 && e < a.E;
    const uint64_t active = ballot(valid);
    uint64_t peers = active;
    for (int b = 0; b < bits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t bal = ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const int rank = __popcll(peers & lt_mask);
    const int cnt = __popcll(peers);
    const bool leader = valid && (rank == cnt - 1);  // last lane of its peer group
    int local = 0;
    for (int w = 0; w < 4; ++w) {
      if (wave == w && valid) {
        const int before = run[e];
        local = before + rank;
        if (leader) run[e] = before + cnt;
      }
      __syncthreads();
    }
    if (valid) {
      const int pos = base[e] + local;
      a.perm[pos] = static_cast<int32_t>(s);
      a.sorted_token[pos] = static_cast<int32_t>(s / a.K);
      a.inv[s] = pos;
      if (a.sorted_w) a.sorted_w[pos] = gs[r];
    } else if (s < s1) {
      a.inv[s] = -1;
    }
  }
}

// The whole dispatch in one workgroup of 1024 threads, for few slots and
// experts (a launch per step costs more than the work there). Each thread
// owns slots t, t + 1024, ... (one per round of 1024): their ids, weights and
// router gaps are loaded once, up front. Per round and wavefront, slots of
// equal id find each other with one ballot per id bit (peer masks), so the
// LDS histogram takes one atomic per (wavefront, id). One exclusive scan of
// packed (count, m-tiles, m-tiles of the second height) per expert gives the
// offsets and both tile tables' starts. A slot's position is its expert's
// running base + the slots of that id in earlier wavefronts of the round +
// its rank among its wavefront's peers: per round the wavefronts' peer
// counts go to LDS and one thread per expert turns them into those bases
// (two barriers a round, the count tables alternating between two buffers).
// Everything up to the positions stays in LDS and registers; the global
// writes all come after the last barrier.
constexpr int kFusedRounds = static_cast<int>(kFusedMaxSlots / 1024);

__device__ __forceinline__ uint64_t block_exscan64_1024(uint64_t v, uint64_t *tmp,
                                                        uint64_t *total) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint64_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  if (w == 0) {
    uint64_t s = lane < 16 ? tmp[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const uint64_t y = __shfl_up(s, off);
      if (lane >= off) s += y;
    }
    if (lane < 16) tmp[lane] = s;
  }
  __syncthreads();
  const uint64_t incl = x + (w ? tmp[w - 1] : 0);
  *total = tmp[15];
  return incl - v;
}

__global__ __launch_bounds__(1024) void dispatch_fused_kernel(ScanArgs a, ScatterArgs sc) {
  __shared__ uint64_t tmp64[16];
  __shared__ int run[kMaxE + 1];
  __shared__ int off[kMaxE + 1];
  __shared__ int start[kMaxE + 1];
  __shared__ int start2[kMaxE + 1];
  __shared__ int wcnt[2][16][kFusedMaxE];
  __shared__ int ntie_total;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int E = a.E;
  const int slots = static_cast<int>(a.slots);
  const int rounds = (slots + 1023) / 1024;
  const bool ties = a.gap && a.n_near_ties;
  const int Tn = ties ? static_cast<int>(a.T) : 0;  // T <= slots
  int ids[kFusedRounds];
  float gs[kFusedRounds], gap[kFusedRounds];
#pragma unroll
  for (int r = 0; r < kFusedRounds; ++r) {
    const int s = r * 1024 + t;
    ids[r] = (r < rounds && s < slots) ? sc.idx[s] : -1;
    gs[r] = (r < rounds && s < slots && sc.sorted_w) ? sc.g[s] : 0.f;
    gap[r] = (r < rounds && s < Tn) ? a.gap[s] : INFINITY;
  }
  for (int e = t; e < E; e += 1024) run[e] = 0;
  if (t == 0) ntie_total = 0;
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rk[kFusedRounds], cn[kFusedRounds];
  __syncthreads();
  int ntie = 0;
#pragma unroll
  for (int r = 0; r < kFusedRounds; ++r) {
    rk[r] = 0;
    cn[r] = 0;
    if (r < rounds) {
      const int e = ids[r];
      const bool valid = e >= 0 && e < E;
      uint64_t peers = ballot(valid);
      for (int b = 0; b < bits; ++b) {
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t bal = ballot(bit);
        peers &= bit ? bal : ~bal;
      }
      rk[r] = __popcll(peers & lt_mask);
      cn[r] = __popcll(peers);
      if (valid && rk[r] == cn[r] - 1) atomicAdd(&run[e], cn[r]);
      ntie += gap[r] < a.tie_eps ? 1 : 0;
    }
  }
  if (ties) {  // near ties: a wavefront sum, one LDS atomic per wavefront
    int v = ntie;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0 && v) atomicAdd(&ntie_total, v);
  }
  __syncthreads();
  // (count, tiles of height bm, tiles of height bm2) per expert, 21 bits each
  const int cnt_t = t < E ? run[t] : 0;
  const uint64_t nt1 = (t < E && a.tiles) ? (cnt_t + a.bm - 1) / a.bm : 0;
  const uint64_t nt2 = (t < E && a.tiles2) ? (cnt_t + a.bm2 - 1) / a.bm2 : 0;
  constexpr uint64_t kM = (1ull << 21) - 1;
  uint64_t tot;
  const uint64_t ex = block_exscan64_1024(static_cast<uint64_t>(cnt_t) | (nt1 << 21) | (nt2 << 42),
                                          tmp64, &tot);
  const int ex_c = static_cast<int>(ex & kM);
  if (t < E) {
    off[t] = ex_c;
    run[t] = ex_c;
    start[t] = static_cast<int>((ex >> 21) & kM);
    start2[t] = static_cast<int>(ex >> 42);
  }
  if (t == 0) {
    off[E] = static_cast<int>(tot & kM);
    start[E] = static_cast<int>((tot >> 21) & kM);
    start2[E] = static_cast<int>(tot >> 42);
  }
  __syncthreads();
  int pos[kFusedRounds];
#pragma unroll
  for (int r = 0; r < kFusedRounds; ++r) {
    pos[r] = -1;
    if (r >= rounds) break;
    int(*wc)[kFusedMaxE] = wcnt[r & 1];
    const int e = ids[r];
    const bool valid = e >= 0 && e < E;
    for (int i = lane; i < E; i += 64) wc[wave][i] = 0;  // this wave's row (in order)
    if (valid && rk[r] == cn[r] - 1) wc[wave][e] = cn[r];
    __syncthreads();
    if (t < E) {  // expert t: bases of its slots per wavefront, then the running base
      int v[16];
#pragma unroll
      for (int w = 0; w < 16; ++w) v[w] = wc[w][t];
      int acc = run[t];
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        wc[w][t] = acc;
        acc += v[w];
      }
      run[t] = acc;
    }
    __syncthreads();
    if (valid) pos[r] = wc[wave][e] + rk[r];
  }

  // global writes
  if (t < E) {
    a.counts[t] = cnt_t;
    a.offsets[t] = ex_c;
  }
  if (t == 0) a.offsets[E] = off[E];
  if (a.tiles) write_tiles(off, E, a.bm, start, a.tiles, a.n_tiles);
  if (a.tiles2) write_tiles(off, E, a.bm2, start2, a.tiles2, a.n_tiles2);
  if (ties && t == 0) *a.n_near_ties = ntie_total;
#pragma unroll
  for (int r = 0; r < kFusedRounds; ++r) {
    if (r >= rounds) break;
    const int s = r * 1024 + t;
    if (pos[r] >= 0) {
      sc.perm[pos[r]] = s;
      sc.sorted_token[pos[r]] = s / sc.K;
      sc.inv[s] = pos[r];
      if (sc.sorted_w) sc.sorted_w[pos[r]] = gs[r];
    } else if (s < slots) {
      sc.inv[s] = -1;
    }
  }
}

// Few experts (E <= 4), one workgroup: thread t owns the R = ceil(slots /
// 1024) consecutive slots [R t, R t + R). Its per-expert counts, 16 bits
// each in one 64-bit word, go through a single block exclusive scan, whose
// result is, per expert, the number of that expert's slots before the
// thread's first one, and whose total holds the per-expert counts; every
// thread then derives the offsets and tile starts of the (at most 4) experts
// itself. Two barriers in all, against two per round of 1024 slots in
// dispatch_fused_kernel.
constexpr int kFewE = 4;

// v[i] for i in [0, kFewE] without a dynamically indexed register array
__device__ __forceinline__ int pick_few(const int (&v)[kFewE + 1], int i) {
  int r = v[0];
#pragma unroll
  for (int j = 1; j <= kFewE; ++j) r = i == j ? v[j] : r;
  return r;
}

__device__ void write_tiles_few(const int (&off)[kFewE + 1], const int (&st)[kFewE + 1], int E,
                                int bm, int32_t *tiles, int32_t *n_tiles) {
  const int total = pick_few(st, E);
  for (int i = threadIdx.x; i < total; i += 1024) {
    int e = 0;
#pragma unroll
    for (int j = 1; j < kFewE; ++j) e += (j < E && st[j] <= i) ? 1 : 0;
    const int se = pick_few(st, e), se1 = pick_few(st, e + 1);
    const int o0 = pick_few(off, e);
    int r0, r1;
    tile_rows(o0, pick_few(off, e + 1) - o0, se1 - se, i - se, bm, &r0, &r1);
    const int gfirst = se + (i - se) / kTileGroup * kTileGroup;
    int32_t *ti = tiles + kTileInts * static_cast<int64_t>(i);
    ti[0] = e;
    ti[1] = r0;
    ti[2] = r1;
    ti[3] = gfirst;
    ti[4] = min(kTileGroup, se1 - gfirst);
  }
  if (threadIdx.x == 0) *n_tiles = total;
}

__global__ __launch_bounds__(1024) void dispatch_few_kernel(ScanArgs a, ScatterArgs sc) {
  __shared__ uint64_t tmp64[16];
  __shared__ int wave_ties[16];
  const int t = threadIdx.x, lane = t & 63;
  const int E = a.E;
  const int slots = static_cast<int>(a.slots);
  const int R = (slots + 1023) / 1024;
  const int s0 = R * t;
  int ids[kFusedRounds];
  float gs[kFusedRounds];
  uint64_t mine = 0;
#pragma unroll
  for (int r = 0; r < kFusedRounds; ++r) {
    const int s = s0 + r;
    const bool in = r < R && s < slots;
    ids[r] = in ? sc.idx[s] : -1;
    gs[r] = (in && sc.sorted_w) ? sc.g[s] : 0.f;
  }
  const bool ties = a.gap && a.n_near_ties;
  if (ties) {  // near ties: per wavefront sums, added up after the scan's barriers
    int n = 0;
    for (int64_t i = t; i < a.T; i += 1024) n += a.gap[i] < a.tie_eps ? 1 : 0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o);
    if (lane == 0) wave_ties[t >> 6] = n;
  }
#pragma unroll
  for (int r = 0; r < kFusedRounds; ++r) {
    const int e = ids[r];
    if (e >= 0 && e < E) mine += 1ull << (16 * e);
  }
  uint64_t tot;
  uint64_t run = block_exscan64_1024(mine, tmp64, &tot);
  int off[kFewE + 1], st1[kFewE + 1], st2[kFewE + 1];
  off[0] = st1[0] = st2[0] = 0;
#pragma unroll
  for (int e = 0; e < kFewE; ++e) {
    const int c = e < E ? static_cast<int>((tot >> (16 * e)) & 0xffff) : 0;
    off[e + 1] = off[e] + c;
    st1[e + 1] = st1[e] + (a.tiles ? (c + a.bm - 1) / a.bm : 0);
    st2[e + 1] = st2[e] + (a.tiles2 ? (c + a.bm2 - 1) / a.bm2 : 0);
  }
#pragma unroll
  for (int r = 0; r < kFusedRounds; ++r) {
    const int s = s0 + r;
    if (r >= R || s >= slots) break;
    const int e = ids[r];
    if (e >= 0 && e < E) {
      const int pos = pick_few(off, e) + static_cast<int>((run >> (16 * e)) & 0xffff);
      run += 1ull << (16 * e);
      sc.perm[pos] = s;
      sc.sorted_token[pos] = s / sc.K;
      sc.inv[s] = pos;
      if (sc.sorted_w) sc.sorted_w[pos] = gs[r];
    } else {
      sc.inv[s] = -1;
    }
  }
  if (t < E) {
    a.counts[t] = pick_few(off, t + 1) - pick_few(off, t);
    a.offsets[t] = pick_few(off, t);
  }
  if (t == 0) {
    a.offsets[E] = pick_few(off, E);
    if (ties) {
      int n = 0;
#pragma unroll
      for (int w = 0; w < 16; ++w) n += wave_ties[w];
      *a.n_near_ties = n;
    }
  }
  if (a.tiles) write_tiles_few(off, st1, E, a.bm, a.tiles, a.n_tiles);
  if (a.tiles2) write_tiles_few(off, st2, E, a.bm2, a.tiles2, a.n_tiles2);
}

// The scan step for fewer than 2^21 slots: per expert its count and its
// m-tile counts for both tile heights, 21 bits each, in one 64-bit block
// scan (the near-tie gaps requested first, so their latency overlaps the
// chunk counts'; the first 64 chunk counts kept in registers for the bases).
// One workgroup of 1024 threads, three barriers against seventeen in
// scan_kernel.
__global__ __launch_bounds__(1024) void scan_packed_kernel(ScanArgs a) {
  __shared__ uint64_t tmp64[16];
  __shared__ int off[kMaxE + 1];
  __shared__ int start[kMaxE + 1];
  __shared__ int start2[kMaxE + 1];
  __shared__ int wave_ties[16];
  const int t = threadIdx.x, lane = t & 63;
  const int E = a.E;
  const int64_t nch = n_chunks(a.slots);
  constexpr int kBatch = 16, kFirst = 64;  // the first 64 chunk counts stay in registers
  const bool ties = a.gap && a.n_near_ties;
  float gv[kBatch];
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const int64_t i = t + 1024 * j;
    gv[j] = (ties && i < a.T) ? a.gap[i] : INFINITY;
  }
  int v0[kFirst];
#pragma unroll
  for (int j = 0; j < kFirst; ++j) v0[j] = (t < E && j < nch) ? a.chunk_hist[j * E + t] : 0;
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < kFirst; ++j) cnt += v0[j];
  for (int64_t c0 = kFirst; t < E && c0 < nch; c0 += kBatch) {
    int v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) v[j] = c0 + j < nch ? a.chunk_hist[(c0 + j) * E + t] : 0;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) cnt += v[j];
  }
  if (ties) {  // per wavefront sums, added after the scan's barriers
    int n = 0;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) n += gv[j] < a.tie_eps ? 1 : 0;
    for (int64_t i0 = t + 1024 * kBatch; i0 < a.T; i0 += 1024 * kBatch) {
      float g[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int64_t i = i0 + 1024 * j;
        g[j] = i < a.T ? a.gap[i] : INFINITY;
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) n += g[j] < a.tie_eps ? 1 : 0;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o);
    if (lane == 0) wave_ties[t >> 6] = n;
  }
  const uint64_t nt1 = (t < E && a.tiles) ? (cnt + a.bm - 1) / a.bm : 0;
  const uint64_t nt2 = (t < E && a.tiles2) ? (cnt + a.bm2 - 1) / a.bm2 : 0;
  constexpr uint64_t kM = (1ull << 21) - 1;
  uint64_t tot;
  const uint64_t ex = block_exscan64_1024(
      static_cast<uint64_t>(t < E ? cnt : 0) | (nt1 << 21) | (nt2 << 42), tmp64, &tot);
  if (t < E) {
    const int ex_c = static_cast<int>(ex & kM);
    off[t] = ex_c;
    start[t] = static_cast<int>((ex >> 21) & kM);
    start2[t] = static_cast<int>(ex >> 42);
    a.counts[t] = cnt;
    a.offsets[t] = ex_c;
    // absolute base of every (chunk, expert) pair (chunk_base may alias
    // chunk_hist: this thread reads each of its elements before writing it)
    int run = ex_c;
#pragma unroll
    for (int j = 0; j < kFirst; ++j)
      if (j < nch) {
        a.chunk_base[j * E + t] = run;
        run += v0[j];
      }
    for (int64_t c0 = kFirst; c0 < nch; c0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) v[j] = c0 + j < nch ? a.chunk_hist[(c0 + j) * E + t] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (c0 + j < nch) {
          a.chunk_base[(c0 + j) * E + t] = run;
          run += v[j];
        }
    }
  }
  if (t == 0) {
    off[E] = static_cast<int>(tot & kM);
    start[E] = static_cast<int>((tot >> 21) & kM);
    start2[E] = static_cast<int>(tot >> 42);
    a.offsets[E] = static_cast<int>(tot & kM);
  }
  __syncthreads();
  if (a.tiles) write_tiles(off, E, a.bm, start, a.tiles, a.n_tiles);
  if (a.tiles2) write_tiles(off, E, a.bm2, start2, a.tiles2, a.n_tiles2);
  if (ties && t == 0) {
    int n = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) n += wave_ties[w];
    *a.n_near_ties = n;
  }
}

// One wavefront per sorted row: out[p, :] = rows[sorted_token[p], :].
__global__ __launch_bounds__(256) void gather_kernel(const uint4 *__restrict__ rows,
                                                     const int32_t *__restrict__ sorted_token,
                                                     int64_t n_rows, int64_t chunks_per_row,
                                                     uint4 *__restrict__ out) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (p >= n_rows) return;
  const int64_t src = sorted_token[p];
  const uint4 *in = rows + src * chunks_per_row;
  uint4 *o = out + p * chunks_per_row;
  for (int64_t i = threadIdx.x & 63; i < chunks_per_row; i += 64) o[i] = in[i];
}

}  // namespace

hipError_t launch_hist(const int32_t *idx, int64_t slots, int E, int32_t *chunk_hist,
                       hipStream_t s) {
  if (slots == 0) return hipSuccess;
  hist_kernel<<<static_cast<unsigned>(n_chunks(slots)), 256, 0, s>>>(idx, slots, E, chunk_hist);
  return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs &a, hipStream_t s) {
  if (a.slots < (int64_t(1) << 21))
    scan_packed_kernel<<<1, 1024, 0, s>>>(a);
  else
    scan_kernel<<<1, 1024, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_tiles(const int32_t *offsets, int E, int bm, int32_t *tiles, int32_t *n_tiles,
                        hipStream_t s) {
  tiles_kernel<<<1, 1024, 0, s>>>(offsets, E, bm, tiles, n_tiles);
  return hipGetLastError();
}

bool dispatch_fused_ok(int64_t slots, int E) {
  return slots <= kFusedMaxSlots && E <= kFusedMaxE;
}

hipError_t launch_dispatch_fused(const ScanArgs &a, const ScatterArgs &sc, hipStream_t s) {
  if (!dispatch_fused_ok(a.slots, a.E)) return hipErrorInvalidValue;
  if (a.E <= kFewE)
    dispatch_few_kernel<<<1, 1024, 0, s>>>(a, sc);
  else
    dispatch_fused_kernel<<<1, 1024, 0, s>>>(a, sc);
  return hipGetLastError();
}

hipError_t launch_scatter(const ScatterArgs &a, hipStream_t s) {
  if (a.slots == 0) return hipSuccess;
  scatter_kernel<<<static_cast<unsigned>(n_chunks(a.slots)), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gather(const void *rows, const int32_t *sorted_token, int64_t n_rows,
                         int64_t row_bytes, void *out, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  gather_kernel<<<static_cast<unsigned>((n_rows + 3) / 4), 256, 0, s>>>(
      static_cast<const uint4 *>(rows), sorted_token, n_rows, row_bytes / 16,
      static_cast<uint4 *>(out));
  return hipGetLastError();
}

}  // namespace moe
