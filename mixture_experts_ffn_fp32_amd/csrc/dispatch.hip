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
//             the near-tie count of the router gaps;
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
  for (int64_t s = s0 + threadIdx.x; s < s1; s += 256) {
    const int e = idx[s];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    chunk_hist[static_cast<int64_t>(blockIdx.x) * E + e] = h[e];
}

// Fill the m-tile table of height bm from offsets held in LDS (1024 threads).
// tile i = {expert, row_begin, row_end, group_first, group_size}; experts
// with no rows get no tile. A group is a run of at most kTileGroup m-tiles
// of one expert (the GEMMs schedule a group's tiles together so they share
// the expert's weight slices in L2).
__device__ void build_tiles(const int *off, int E, int bm, int *start, int *tmp,
                            int32_t *tiles, int32_t *n_tiles) {
  const int t = threadIdx.x;
  int nt = 0;
  if (t < E) nt = (off[t + 1] - off[t] + bm - 1) / bm;
  int total;
  const int ex = block_exscan_1024(nt, tmp, &total);
  if (t < E) start[t] = ex;
  if (t == 0) start[E] = total;
  __syncthreads();
  for (int i = t; i < total; i += 1024) {
    int lo = 0, hi = E;  // find e with start[e] <= i < start[e+1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (start[mid] <= i) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int r0 = off[e] + (i - start[e]) * bm;
    const int gfirst = start[e] + (i - start[e]) / kTileGroup * kTileGroup;
    int32_t *ti = tiles + kTileInts * static_cast<int64_t>(i);
    ti[0] = e;
    ti[1] = r0;
    ti[2] = min(r0 + bm, off[e + 1]);
    ti[3] = gfirst;
    ti[4] = min(kTileGroup, start[e + 1] - gfirst);
  }
  if (t == 0) *n_tiles = total;
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
  for (int64_t r0 = s0; r0 < s1; r0 += 256) {
    const int64_t s = r0 + tid;
    int e = -1;
    if (s < s1) e = a.idx[s];
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
      if (a.sorted_w) a.sorted_w[pos] = a.g[s];
    } else if (s < s1) {
      a.inv[s] = -1;
    }
  }
}

// The whole dispatch in one workgroup of 1024 threads, for few slots and
// experts (a launch per step costs more than the work there). Each thread
// owns slots t, t + 1024, ... (one per round of 1024): their ids, weights and
// the router gaps are loaded once, up front. Per round and wavefront, slots
// of equal id find each other with one ballot per id bit (peer masks), so
// the LDS histogram takes one atomic per (wavefront, id), and a slot's
// position is its expert's running base + the slots of that id in earlier
// wavefronts of the round (per-wavefront peer counts in LDS) + its rank among
// its wavefront's peers. Scan, m-tile tables and near-tie count as in
// scan_kernel.
constexpr int kFusedRounds = static_cast<int>(kFusedMaxSlots / 1024);

__global__ __launch_bounds__(1024) void dispatch_fused_kernel(ScanArgs a, ScatterArgs sc) {
  __shared__ int tmp[1024];
  __shared__ int run[kMaxE + 1];
  __shared__ int off[kMaxE + 1];
  __shared__ int start[kMaxE + 1];
  __shared__ int wcnt[16][kFusedMaxE];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int E = a.E;
  const int rounds = static_cast<int>((a.slots + 1023) / 1024);
  int ids[kFusedRounds];
  float gs[kFusedRounds];
#pragma unroll
  for (int r = 0; r < kFusedRounds; ++r) {
    const int64_t s = static_cast<int64_t>(r) * 1024 + t;
    ids[r] = (r < rounds && s < a.slots) ? sc.idx[s] : -1;
    gs[r] = (r < rounds && s < a.slots && sc.sorted_w) ? sc.g[s] : 0.f;
  }
  int ntie = 0;
  if (a.gap && a.n_near_ties)
    for (int64_t i = t; i < a.T; i += 1024) ntie += (a.gap[i] < a.tie_eps) ? 1 : 0;
  for (int e = t; e < E; e += 1024) run[e] = 0;
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rk[kFusedRounds], cn[kFusedRounds];
  __syncthreads();
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
    }
  }
  __syncthreads();
  const int cnt_t = t < E ? run[t] : 0;
  int total;
  const int ex = block_exscan_1024(cnt_t, tmp, &total);
  if (t < E) {
    off[t] = ex;
    run[t] = ex;
    a.counts[t] = cnt_t;
    a.offsets[t] = ex;
  }
  if (t == 0) {
    off[E] = total;
    a.offsets[E] = total;
  }
  __syncthreads();
  if (a.tiles) build_tiles(off, E, a.bm, start, tmp, a.tiles, a.n_tiles);
  __syncthreads();
  if (a.tiles2) build_tiles(off, E, a.bm2, start, tmp, a.tiles2, a.n_tiles2);
  __syncthreads();
  if (a.gap && a.n_near_ties) {
    int tot;
    block_exscan_1024(ntie, tmp, &tot);
    if (t == 0) *a.n_near_ties = tot;
  }
#pragma unroll
  for (int r = 0; r < kFusedRounds; ++r) {
    if (r >= rounds) break;
    const int64_t s = static_cast<int64_t>(r) * 1024 + t;
    const int e = ids[r];
    const bool valid = e >= 0 && e < E;
    for (int i = lane; i < E; i += 64) wcnt[wave][i] = 0;  // this wave's row (in order)
    if (valid && rk[r] == cn[r] - 1) wcnt[wave][e] = cn[r];
    __syncthreads();
    int pos = 0;
    if (valid) {
      int pre = 0;
      for (int w = 0; w < wave; ++w) pre += wcnt[w][e];
      pos = run[e] + pre + rk[r];
    }
    __syncthreads();  // every read of run[] and wcnt[] of this round is done
    if (t < E) {
      int add = 0;
#pragma unroll
      for (int w = 0; w < 16; ++w) add += wcnt[w][t];
      run[t] += add;
    }
    if (valid) {
      sc.perm[pos] = static_cast<int32_t>(s);
      sc.sorted_token[pos] = static_cast<int32_t>(s / sc.K);
      sc.inv[s] = pos;
      if (sc.sorted_w) sc.sorted_w[pos] = gs[r];
    } else if (s < a.slots) {
      sc.inv[s] = -1;
    }
    __syncthreads();  // run[] updated before the next round reads it
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
