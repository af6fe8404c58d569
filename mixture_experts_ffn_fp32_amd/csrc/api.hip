// C ABI of libmoe.so: argument checks, workspace layout and the launch
// sequence of each entry point. Every step of the layer runs in this
// library's HIP kernels; the host only validates and enqueues.
#include <stddef.h>
#include <stdint.h>

#include <initializer_list>
#include <mutex>

#include "kernels.h"
#include "moe.h"

// Workspace of moe_forward_noalloc: a file-scope device array, one copy on
// each GPU the library runs on. In host code `scratch` names a host-side
// stand-in, not a device address: the address of the current device's copy
// comes from hipGetSymbolAddress (taken once per device, below) and only
// that pointer is ever handed to kernels.
static __device__ __align__(256) char scratch[MOE_SCRATCH_BYTES];

namespace {

using namespace moe;

constexpr float kTieEps = 1e-5f;
constexpr int kMaxLatent = 16384;

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct Layout {
  size_t wsplit, logits;
  size_t idx, g, gap, counts, offsets, chunk, perm, stok, inv, sw, tiles, ntiles, tiles2,
      ntiles2, ntie;
  size_t z, h, y, hsh, sh, r;
  size_t qb_top, qb_diff, qb_q;  // QuantileBalancer (sigmoid routing only)
  size_t loss;                   // router-loss partial sums
  size_t total;
  int64_t max_tiles;
};

int64_t grouped_tile_bound(int64_t rows, int64_t E, int bm) {
  return rows / bm + (rows < E ? rows : E) + 1;
}

bool merged_plan(const moe_desc *d);
bool shared_rows_f32(const moe_desc *d);

Layout layout_of(const moe_desc *d) {
  Layout L{};
  const int64_t T = d->T, K = d->top_k, E = d->n_experts, rows = T * K;
  const size_t es = d->act_dtype == MOE_BF16 ? 2 : 4;
  const int64_t de = d->latent ? d->latent : d->d_model;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  const int bf = d->act_dtype == MOE_BF16;
  L.wsplit = take(router_split_bytes(E, d->d_model, bf));
  L.logits = take(router_logit_bytes(T, E, d->d_model, bf));
  L.idx = take(rows * 4);
  L.g = take(rows * 4);
  L.gap = take(T * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.chunk = take(static_cast<size_t>(n_chunks(rows)) * E * 4);
  L.perm = take(rows * 4);
  L.stok = take(rows * 4);
  L.inv = take(rows * 4);
  L.sw = take(rows * 4);
  L.max_tiles = grouped_tile_bound(rows, E, 16);  // smallest tile height in use
  L.tiles = take(static_cast<size_t>(L.max_tiles) * kTileInts * 4);
  L.ntiles = take(4);
  L.tiles2 = take(static_cast<size_t>(L.max_tiles) * kTileInts * 4);
  L.ntiles2 = take(4);
  L.ntie = take(4);
  L.z = d->latent ? take(T * d->latent * es) : 0;
  L.h = take(rows * d->d_ff * es);
  L.y = take(rows * de * es);
  L.hsh = d->d_shared ? take(T * d->d_shared * es) : 0;
  L.sh = shared_rows_f32(d) ? take(T * d->d_model * 4) : 0;  // fp32
  L.r = d->latent ? take(T * d->latent * es) : 0;
  if (d->route_mode == MOE_ROUTE_SIGMOID_BIAS) {
    L.qb_top = take(T * (K + 1) * 4);
    L.qb_diff = take(T * E * 4);
    L.qb_q = take(E * 4);
  }
  L.loss = take(static_cast<size_t>(router_loss_chunks(T)) * (E + 1) * 4);
  L.total = o;
  return L;
}

int check_desc(const moe_desc *d) {
  if (!d) return MOE_ERR_NULL;
  if (d->act_dtype != MOE_F32 && d->act_dtype != MOE_BF16) return MOE_ERR_MODE;
  if (d->route_mode < MOE_ROUTE_TOPK_SOFTMAX || d->route_mode > MOE_ROUTE_SIGMOID_BIAS)
    return MOE_ERR_MODE;
  if (d->has_rmsnorm && !d->latent) return MOE_ERR_MODE;
  if (d->T < 0 || d->d_model <= 0 || d->d_ff <= 0 || d->n_experts < 1 || d->n_experts > 1024)
    return MOE_ERR_SHAPE;
  if (d->top_k < 1 || d->top_k > 16 || d->top_k > d->n_experts) return MOE_ERR_SHAPE;
  if (d->d_shared < 0 || d->latent < 0 || d->latent > kMaxLatent) return MOE_ERR_SHAPE;
  if (d->d_model % 8 || d->d_ff % 8 || d->d_shared % 8 || d->latent % 8) return MOE_ERR_SHAPE;
  if (d->T * static_cast<int64_t>(d->top_k) > 0x7FFFFFFF) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// Kernel and tile shape of each grouped expert GEMM. Each has its own m-tile
// table unless the two tile heights agree.
struct GemmPlan {
  int v2, cfg;
  int bm() const { return v2 ? gemm2_bm(cfg) : tile_bm(cfg); }
};
struct Plan {
  GemmPlan gu, dn;  // gate/up, down
  bool merged;      // the shared experts' GEMMs run inside the grouped launches
  bool shared_table() const { return gu.bm() == dn.bm(); }
};

// The pipelined kernel when it applies (bf16, K a multiple of 32, 32-bit
// operand extents): 32 x 256 tiles streaming the weights for ~32 rows per
// expert or fewer (decode), else the tile gemm2_pick chooses; otherwise the
// generic kernel: 16-row tiles for few rows per expert, 128x128 otherwise
// (128x64 for bf16 down projections that would give fewer than 256
// workgroups).
// (a_rows: rows the GEMM's A operand spans; the pipelined kernel addresses
// A and each expert's B with 32-bit offsets.)
GemmPlan plan_one(int64_t rows, int64_t E, int64_t K, int64_t n_out, int glu, int bf,
                  int64_t a_rows) {
  constexpr int64_t kLim = int64_t(1) << 32;
  const bool small_extent = a_rows * K * 2 < kLim && (n_out + 256) * K * 2 < kLim;
  const bool v2 = bf && K % 32 == 0 && n_out % 8 == 0 && small_extent;
  if (rows <= 32 * E)  // ~32 rows per expert or fewer: weight streaming
    return v2 ? GemmPlan{1, TILE2_32x256_D2} : GemmPlan{0, TILE_SMALL_M};
  if (v2) return {1, gemm2_pick(rows, E, K, n_out, glu)};
  const int64_t mt = rows / tile_bm(TILE_LARGE) + (rows < E ? rows : E);
  if (!bf || glu || mt * tile_count(TILE_LARGE, 1, n_out, glu) >= 256) return {0, TILE_LARGE};
  return {0, TILE_TALL_N64};  // few down tiles (narrow model, few experts)
}

// Layers too small for 256x256 grouped tiles leave CUs idle in every GEMM
// launch; there the shared experts' gate/up and down GEMMs join the grouped
// launches as second problems (same tile), and the combine becomes a
// gather-sum that adds their output.
Plan plan_grouped(const moe_desc *d) {
  const int64_t rows = d->T * d->top_k, E = d->n_experts;
  const int64_t de = d->latent ? d->latent : d->d_model;
  const int bf = d->act_dtype == MOE_BF16;
  Plan pl{plan_one(rows, E, de, d->d_ff, 1, bf, rows),  // A: T tokens or T*K gathered rows
          plan_one(rows, E, d->d_ff, de, 0, bf, rows), false};
  const int64_t T = d->T, dm = d->d_model, ds = d->d_shared;
  constexpr int64_t kLim = int64_t(1) << 32;
  if (!d->latent && ds > 0 && bf && pl.gu.v2 && pl.dn.v2 && pl.gu.cfg != TILE2_256x256_TALLW &&
      dm % 32 == 0 && ds % 32 == 0 && T * dm * 2 < kLim && T * ds * 2 < kLim &&
      (ds + 256) * dm * 2 < kLim && (dm + 256) * ds * 2 < kLim) {
    pl.merged = true;
    if (rows > 32 * E) {  // (weight-streaming tiles stay as they are)
      pl.gu.cfg = gemm2_pick(rows, E, dm, d->d_ff, 1, T, ds);
      pl.dn.cfg = gemm2_pick(rows, E, d->d_ff > ds ? d->d_ff : ds, dm, 0, T, dm);
    }
  }
  return pl;
}

bool merged_plan(const moe_desc *d) { return plan_grouped(d).merged; }

// The shared experts' down projection goes to fp32 rows (sh) that the
// combine kernel adds to the routed rows — on merged plans, and on the other
// non-latent bf16 layers with more than 64 tokens, where the pipelined
// kernel's gather-sum epilogue (K dependent row loads per output chunk, on
// one workgroup per CU) measured slower than a separate combine pass with a
// wavefront per token.
bool shared_rows_f32(const moe_desc *d) {
  return merged_plan(d) ||
         (!d->latent && d->d_shared > 0 && d->act_dtype == MOE_BF16 && d->T > 64);
}

hipError_t run_grouped(const GemmArgs &a, int epi, const GemmPlan &pl, int bf, hipStream_t s) {
  if (!pl.v2) return launch_gemm(a, epi, pl.cfg, bf, s);
  if (!gemm2_applicable(a, epi)) return hipErrorInvalidValue;  // the plan checked this
  return launch_gemm2(a, epi, pl.cfg, s);
}

// m-tile tables of the two grouped GEMMs (gate/up, down)
struct Tables {
  const int32_t *gu, *gu_n, *dn, *dn_n;
};

struct Probe {
  const moe_probe *p;
  hipStream_t s;
  void begin(int stage) const {
    if (p && p->stage == stage) (void)hipEventRecord(static_cast<hipEvent_t>(p->ev_begin), s);
  }
  void end(int stage) const {
    if (p && p->stage == stage) (void)hipEventRecord(static_cast<hipEvent_t>(p->ev_end), s);
  }
  // passes of a GEMM stage to enqueue (repeat > 1 on the probed stage only)
  int reps(int stage) const {
    return (p && p->stage == stage && p->repeat > 1) ? p->repeat : 1;
  }
};

#define MOE_TRY(expr)                          \
  do {                                         \
    if ((expr) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

// Grouped SwiGLU over the sorted rows: GEMM 1 (gate/up + SiLU*up) into h,
// GEMM 2 (down, times row_scale) into y.
int expert_gemms(const moe_desc *d, const moe_weights *w, const void *rows,
                 const int32_t *row_index, const Tables &tb, const Plan &pl,
                 const float *row_scale, void *h, void *y, const Probe &pr, hipStream_t s) {
  const int64_t rows_n = d->T * d->top_k;
  const int de = d->latent ? d->latent : d->d_model;
  const int bf = d->act_dtype == MOE_BF16;
  GemmArgs a{};
  a.a = rows;
  a.lda = de;
  a.a_rows = row_index;
  a.b0 = w->w_gate;
  a.b1 = w->w_up;
  a.ldb = de;
  a.b_stride = static_cast<int64_t>(d->d_ff) * de;
  a.K = de;
  a.N = d->d_ff;
  a.a_extent = row_index ? d->T : rows_n;  // tokens, or rows already gathered
  a.tiles = tb.gu;
  a.n_tiles = tb.gu_n;
  a.max_mtiles = grouped_tile_bound(rows_n, d->n_experts, pl.gu.bm());
  a.out = h;
  a.ldo = d->d_ff;
  pr.begin(MOE_STAGE_EXPERT_GATE_UP);
  for (int r = 0; r < pr.reps(MOE_STAGE_EXPERT_GATE_UP); ++r)
    MOE_TRY(run_grouped(a, EPI_SWIGLU, pl.gu, bf, s));
  pr.end(MOE_STAGE_EXPERT_GATE_UP);

  GemmArgs b{};
  b.a = h;
  b.lda = d->d_ff;
  b.b0 = w->w_down;
  b.ldb = d->d_ff;
  b.b_stride = static_cast<int64_t>(de) * d->d_ff;
  b.K = d->d_ff;
  b.N = de;
  b.a_extent = rows_n;
  b.tiles = tb.dn;
  b.n_tiles = tb.dn_n;
  b.max_mtiles = grouped_tile_bound(rows_n, d->n_experts, pl.dn.bm());
  b.out = y;
  b.ldo = de;
  b.row_scale = row_scale;
  pr.begin(MOE_STAGE_EXPERT_DOWN);
  for (int r = 0; r < pr.reps(MOE_STAGE_EXPERT_DOWN); ++r)
    MOE_TRY(run_grouped(b, EPI_SCALE, pl.dn, bf, s));
  pr.end(MOE_STAGE_EXPERT_DOWN);
  return MOE_OK;
}

// The shared experts' first GEMM: H_shared = SiLU(x Ws_gate^T) * (x Ws_up^T).
int shared_gate_up(const moe_desc *d, const moe_weights *w, const void *x, char *ws,
                   const Layout &L, const Probe &pr, hipStream_t s) {
  const int bf = d->act_dtype == MOE_BF16;
  const int dm = d->d_model;
  void *hsh = ws + L.hsh;
  if (d->d_shared) {
    GemmArgs a{};
    a.a = x;
    a.lda = dm;
    a.b0 = w->ws_gate;
    a.b1 = w->ws_up;
    a.ldb = dm;
    a.K = dm;
    a.N = d->d_shared;
    a.M = d->T;
    a.out = hsh;
    a.ldo = d->d_shared;
    pr.begin(MOE_STAGE_SHARED_GATE_UP);
    for (int r = 0; r < pr.reps(MOE_STAGE_SHARED_GATE_UP); ++r)
      MOE_TRY(launch_dense(a, EPI_SWIGLU, bf, s));
    pr.end(MOE_STAGE_SHARED_GATE_UP);
  }
  return MOE_OK;
}

// Shared experts + combine (+ latent RMSNorm and up-projection) into out;
// with have_hsh the shared experts' first GEMM has already run.
int shared_combine(const moe_desc *d, const moe_weights *w, const void *x, const void *y,
                   const int32_t *inv, void *out, char *ws, const Layout &L, const Probe &pr,
                   hipStream_t s, bool have_hsh = false) {
  const int64_t T = d->T;
  const int bf = d->act_dtype == MOE_BF16;
  const int dm = d->d_model;
  void *hsh = ws + L.hsh;
  if (!have_hsh) {
    const int rc = shared_gate_up(d, w, x, ws, L, pr, s);
    if (rc) return rc;
  }
  pr.begin(MOE_STAGE_COMBINE);
  if (!d->latent) {
    if (d->d_shared) {
      GemmArgs c{};
      c.a = hsh;
      c.lda = d->d_shared;
      c.b0 = w->ws_down;
      c.ldb = d->d_shared;
      c.K = d->d_shared;
      c.N = dm;
      c.M = T;
      if (shared_rows_f32(d)) {  // fp32 rows, then the combine kernel adds them
        float *sh = reinterpret_cast<float *>(ws + L.sh);
        c.out = sh;
        c.ldo = dm;
        c.out_f32 = 1;
        MOE_TRY(launch_dense(c, EPI_SCALE, bf, s));
        MOE_TRY(launch_combine_sum(y, inv, T, d->top_k, dm, out, bf, s, sh));
      } else {
        c.out = out;
        c.ldo = dm;
        c.y = y;
        c.ldy = dm;
        c.inv = inv;
        c.topk = d->top_k;
        MOE_TRY(launch_dense(c, EPI_COMBINE, bf, s));
      }
    } else {
      MOE_TRY(launch_combine_sum(y, inv, T, d->top_k, dm, out, bf, s));
    }
  } else {
    void *r = ws + L.r;
    MOE_TRY(launch_combine_latent(y, inv, T, d->top_k, d->latent, d->has_rmsnorm, d->rms_eps,
                                  w->rms_gamma, r, bf, s));
    GemmArgs c{};
    if (d->d_shared) {
      c.a = hsh;
      c.lda = d->d_shared;
      c.b0 = w->ws_down;
      c.ldb = d->d_shared;
      c.K = d->d_shared;
      c.a2 = r;
      c.lda2 = d->latent;
      c.b2 = w->w_lat_up;
      c.ldb2 = d->latent;
      c.K2 = d->latent;
    } else {
      c.a = r;
      c.lda = d->latent;
      c.b0 = w->w_lat_up;
      c.ldb = d->latent;
      c.K = d->latent;
    }
    c.N = dm;
    c.M = T;
    c.out = out;
    c.ldo = dm;
    MOE_TRY(launch_dense(c, EPI_STORE, bf, s));
  }
  pr.end(MOE_STAGE_COMBINE);
  return MOE_OK;
}

// Counting-sort dispatch: one workgroup for few slots and experts, else
// histogram, scan and scatter launches.
hipError_t run_dispatch(const ScanArgs &sa, const ScatterArgs &sc, hipStream_t s) {
  if (dispatch_fused_ok(sa.slots, sa.E)) return launch_dispatch_fused(sa, sc, s);
  hipError_t e = launch_hist(sc.idx, sa.slots, sa.E, const_cast<int32_t *>(sa.chunk_hist), s);
  if (e != hipSuccess) return e;
  if ((e = launch_scan(sa, s)) != hipSuccess) return e;
  return launch_scatter(sc, s);
}

// Merged plan: grouped gate/up + shared gate/up in one launch, grouped down
// + shared down (into sh, fp32) in one launch, then out = sh + the routed
// rows.
int merged_gemms(const moe_desc *d, const moe_weights *w, const void *x, const void *rows,
                 const int32_t *row_index, const Tables &tb, const Plan &pl,
                 const float *row_scale, const int32_t *inv, void *out, char *ws,
                 const Layout &L, const Probe &pr, hipStream_t s) {
  const int64_t T = d->T, rows_n = T * d->top_k;
  const int dm = d->d_model, ds = d->d_shared;
  void *h = ws + L.h, *y = ws + L.y, *hsh = ws + L.hsh, *sh = ws + L.sh;
  GemmArgs a{};  // routed gate/up
  a.a = rows;
  a.lda = dm;
  a.a_rows = row_index;
  a.b0 = w->w_gate;
  a.b1 = w->w_up;
  a.ldb = dm;
  a.b_stride = static_cast<int64_t>(d->d_ff) * dm;
  a.K = dm;
  a.N = d->d_ff;
  a.a_extent = row_index ? T : rows_n;
  a.tiles = tb.gu;
  a.n_tiles = tb.gu_n;
  a.max_mtiles = grouped_tile_bound(rows_n, d->n_experts, pl.gu.bm());
  a.out = h;
  a.ldo = d->d_ff;
  GemmArgs sa{};  // shared gate/up
  sa.a = x;
  sa.lda = dm;
  sa.b0 = w->ws_gate;
  sa.b1 = w->ws_up;
  sa.ldb = dm;
  sa.K = dm;
  sa.N = ds;
  sa.M = T;
  sa.out = hsh;
  sa.ldo = ds;
  if (!gemm2_applicable(a, EPI_SWIGLU) || !gemm2_applicable(sa, EPI_SWIGLU)) return MOE_ERR_HIP;
  pr.begin(MOE_STAGE_EXPERT_GATE_UP);
  for (int r = 0; r < pr.reps(MOE_STAGE_EXPERT_GATE_UP); ++r)
    MOE_TRY(launch_gemm2(a, EPI_SWIGLU, pl.gu.cfg, s, &sa));
  pr.end(MOE_STAGE_EXPERT_GATE_UP);

  GemmArgs b{};  // routed down, times the routing weight
  b.a = h;
  b.lda = d->d_ff;
  b.b0 = w->w_down;
  b.ldb = d->d_ff;
  b.b_stride = static_cast<int64_t>(dm) * d->d_ff;
  b.K = d->d_ff;
  b.N = dm;
  b.a_extent = rows_n;
  b.tiles = tb.dn;
  b.n_tiles = tb.dn_n;
  b.max_mtiles = grouped_tile_bound(rows_n, d->n_experts, pl.dn.bm());
  b.out = y;
  b.ldo = dm;
  b.row_scale = row_scale;
  GemmArgs sb{};  // shared down (weight 1)
  sb.a = hsh;
  sb.lda = ds;
  sb.b0 = w->ws_down;
  sb.ldb = ds;
  sb.K = ds;
  sb.N = dm;
  sb.M = T;
  sb.out = sh;
  sb.ldo = dm;
  sb.out_f32 = 1;  // fp32, added to the routed rows in fp32 by the combine
  if (!gemm2_applicable(b, EPI_SCALE) || !gemm2_applicable(sb, EPI_SCALE)) return MOE_ERR_HIP;
  pr.begin(MOE_STAGE_EXPERT_DOWN);
  for (int r = 0; r < pr.reps(MOE_STAGE_EXPERT_DOWN); ++r)
    MOE_TRY(launch_gemm2(b, EPI_SCALE, pl.dn.cfg, s, &sb));
  pr.end(MOE_STAGE_EXPERT_DOWN);

  pr.begin(MOE_STAGE_COMBINE);
  MOE_TRY(launch_combine_sum(y, inv, T, d->top_k, dm, out, 1, s, static_cast<const float *>(sh)));
  pr.end(MOE_STAGE_COMBINE);
  return MOE_OK;
}

// ------------------------------------------------------------ backward
// Workspace of moe_backward beyond the forward layout: transposed weights of
// the active experts, per-row fp32 pre-activations and gradients, the
// activations in expert-contiguous, 64-padded columns for the K-grouped
// weight-gradient GEMMs, and (latent layers) the recomputed routed sum and
// the projections' buffers. de is the routed width (d_model, or L).
// Which backward products read the weights in place, K-major on the
// pipelined kernel (bf16), instead of transposed copies: dh (W_down and the
// shared W_down), dX (W_gate and W_up as two K segments: d_ff and d_shared
// multiples of 64) and the latent projections. The expert weights are read
// in place wherever the kernel applies: with its stage loads out of the
// compiler's LDS tracking, the transposing reads cost little per stage and
// the copies cost more on every layer measured (medium 5.96 -> 5.62 ms,
// latent 3.93 -> 3.82, small 0.384 -> 0.377, large prefill level); the
// latent projections only when the layer streams its weights (64 rows per
// expert or fewer; elsewhere level). The shapes restate the products
// moe_backward runs.
struct KmajorUse {
  bool dh, dx, lat;
};
KmajorUse kmajor_use(const moe_desc *d) {
  KmajorUse u{false, false, false};
  if (d->act_dtype != MOE_BF16) return u;
  const int64_t T = d->T, rows = T * d->top_k, E = d->n_experts;
  const int dm = d->d_model, f = d->d_ff, ds = d->d_shared, Lt = d->latent;
  const int de = Lt ? Lt : dm;
  const bool stream = rows <= 64 * E;
  auto prod = [](int64_t M, int64_t a_extent, int64_t lda, int K, int N, int64_t ldb) {
    GemmArgs g{};
    g.M = M;
    g.a_extent = a_extent;
    g.lda = lda;
    g.K = K;
    g.N = N;
    g.ldb = ldb;
    g.ldo = N;
    g.b_kmajor = 1;
    return g;
  };
  static const char kSegment = 0;
  auto second = [](GemmArgs g, int64_t lda2, int K2, int64_t ldb2) {
    g.a2 = &kSegment;  // (only its presence matters here)
    g.lda2 = lda2;
    g.K2 = K2;
    g.ldb2 = ldb2;
    return g;
  };
  auto ok = [](const GemmArgs &g) { return gemm2_applicable(g, EPI_STORE_F32); };
  u.dh = ok(prod(rows, T, de, de, f, f)) && (!ds || ok(prod(T, T, dm, dm, ds, ds)));
  u.dx = f % 64 == 0 && ds % 64 == 0 &&
         ok(second(prod(rows, rows, 2 * f, f, de, de), 2 * f, f, de)) &&
         (!ds || ok(second(prod(T, T, 2 * ds, ds, dm, dm), 2 * ds, ds, dm)));
  u.lat = Lt && stream && ok(prod(T, T, dm, dm, Lt, Lt)) && ok(prod(T, T, Lt, Lt, dm, dm));
  return u;
}

struct BwdLayout {
  size_t poff, kt1, kn1, kt2, kn2, tiles, ntiles;
  size_t wguT, wdT, wsguT, wsdT;
  size_t apre, upre, dhu, h, dau, dg, dr, dxs, dwr_part;
  size_t apre_s, upre_s, dhu_s, h_s, dau_s, dxsh;
  size_t xsT, dysT, daT, duT, hT, xT, dyT, dashT, dushT, hshT;
  // latent
  size_t wluT, wldT, yf, R, rinv, Rp, dRp, dR, dz, dxl, gpart, RpT, dzT;
  size_t total;
  int64_t RP, TP, kt_cap;
};

BwdLayout bwd_layout_of(const moe_desc *d) {
  BwdLayout B{};
  const int64_t T = d->T, K = d->top_k, E = d->n_experts, rows = T * K;
  const int64_t dm = d->d_model, f = d->d_ff, ds = d->d_shared, Lt = d->latent;
  const int64_t de = Lt ? Lt : dm;
  const int64_t es = d->act_dtype == MOE_BF16 ? 2 : 4;  // act element size
  size_t o = layout_of(d).total;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  B.RP = (rows + 63) / 64 * 64 + 64 * E;  // padded expert columns (upper bound)
  B.TP = (T + 63) / 64 * 64;
  B.kt_cap = E * ((f > de ? f : de) + 63) / 64 + 1;
  B.poff = take((E + 1) * 4);
  B.kt1 = take(B.kt_cap * kTileInts * 4);
  B.kn1 = take(4);
  B.kt2 = take(B.kt_cap * kTileInts * 4);
  B.kn2 = take(4);
  B.tiles = take(static_cast<size_t>(grouped_tile_bound(rows, E, 32)) * kTileInts * 4);
  B.ntiles = take(4);
  const KmajorUse ku = kmajor_use(d);  // weights read in place need no copy
  B.wguT = ku.dx ? 0 : take(E * de * 2 * f * es);  // [E, de, 2 f]: W_gate^T | W_up^T
  B.wdT = ku.dh ? 0 : take(E * f * de * es);       // [E, f, de]
  B.wsguT = ku.dx ? 0 : take(dm * 2 * ds * es);
  B.wsdT = ku.dh ? 0 : take(ds * dm * es);
  B.apre = take(rows * f * 4);
  B.upre = take(rows * f * 4);
  B.dhu = take(rows * f * 4);
  B.h = take(rows * f * es);
  B.dau = take(rows * 2 * f * es);
  B.dg = take(rows * 4);
  B.dr = take(rows * 4);
  B.dxs = take(rows * de * 4);
  B.dwr_part = take(dwr_part_bytes(static_cast<int>(E), static_cast<int>(dm)));
  B.apre_s = take(T * ds * 4);
  B.upre_s = take(T * ds * 4);
  B.dhu_s = take(T * ds * 4);
  B.h_s = take(T * ds * es);
  B.dau_s = take(T * 2 * ds * es);
  B.dxsh = take(T * dm * 4);
  B.xsT = take(de * B.RP * es);
  B.dysT = take(de * B.RP * es);
  B.daT = take(f * B.RP * es);
  B.duT = take(f * B.RP * es);
  B.hT = take(f * B.RP * es);
  B.xT = take(dm * B.TP * es);
  B.dyT = take(dm * B.TP * es);
  B.dashT = take(ds * B.TP * es);
  B.dushT = take(ds * B.TP * es);
  B.hshT = take(ds * B.TP * es);
  if (Lt) {
    B.wluT = ku.lat ? 0 : take(Lt * dm * es);
    B.wldT = ku.lat ? 0 : take(dm * Lt * es);
    B.yf = take(rows * Lt * 4);
    B.R = take(T * Lt * 4);
    B.rinv = take(T * 4);
    B.Rp = take(T * Lt * es);
    B.dRp = take(T * Lt * 4);
    B.dR = take(T * Lt * es);
    B.dz = take(T * Lt * es);
    B.dxl = take(T * dm * 4);
    B.gpart = take(static_cast<size_t>(colsum_blocks(T)) * Lt * 4);
    B.RpT = take(Lt * B.TP * es);
    B.dzT = take(Lt * B.TP * es);
  }
  B.total = o;
  return B;
}

int check_backward(const moe_desc *d) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (d->d_model % 32 || d->d_ff % 32 || d->d_shared % 32 || d->latent % 32) return MOE_ERR_SHAPE;
  constexpr int64_t kLim = int64_t(1) << 32;  // 32-bit operand offsets of the GEMMs
  const int64_t T = d->T, rows = T * d->top_k, E = d->n_experts;
  const int64_t dm = d->d_model, f = d->d_ff, ds = d->d_shared;
  const int64_t de = d->latent ? d->latent : dm, wm = dm > de ? dm : de;
  const int64_t RP = (rows + 63) / 64 * 64 + 64 * E, mx = (wm > f ? wm : f) + 256;
  const int64_t TP = (T + 63) / 64 * 64;
  if (T * wm * 2 >= kLim || rows * 2 * f * 2 >= kLim || mx * RP * 2 >= kLim ||
      (f + 256) * 2 * f * 2 >= kLim || mx * 2 * (ds > f ? ds : f) * 2 >= kLim ||
      T * 2 * ds * 2 >= kLim || mx * TP * 2 >= kLim || mx * wm * 2 >= kLim)
    return MOE_ERR_SHAPE;
  return MOE_OK;
}

// Device arrays the kernels move in 16-byte chunks (activations, weights,
// routed rows, outputs, gradients, workspaces) must be 16-byte aligned, as
// torch's allocations are. NULL passes (presence is checked separately).
bool aligned16(std::initializer_list<const void *> ps) {
  for (const void *p : ps)
    if (reinterpret_cast<uintptr_t>(p) & 15) return false;
  return true;
}
bool weights_aligned(const moe_weights *w) {
  return aligned16({w->w_router, w->bias, w->rms_gamma, w->w_gate, w->w_up, w->w_down,
                    w->ws_gate, w->ws_up, w->ws_down, w->w_lat_down, w->w_lat_up});
}

int check_expert_weights(const moe_desc *d, const moe_weights *w) {
  if (!w || !w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_NULL;
  return MOE_OK;
}

int check_combine_weights(const moe_desc *d, const moe_weights *w) {
  if (!w) return MOE_ERR_NULL;
  if (d->d_shared && (!w->ws_gate || !w->ws_up || !w->ws_down)) return MOE_ERR_NULL;
  if (d->latent && !w->w_lat_up) return MOE_ERR_NULL;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char *moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "invalid shape";
    case MOE_ERR_MODE: return "invalid dtype or mode combination";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP kernel launch failed";
    case MOE_ERR_SCRATCH:
      return "layer needs more than the static scratch (MOE_SCRATCH_BYTES), or the stream is "
             "on another device";
  }
  return "unknown status";
}

const char *moe_stage_name(int stage) {
  static const char *names[MOE_STAGE_COUNT] = {"route", "dispatch", "latent_down",
                                               "expert_gate_up", "expert_down",
                                               "shared_gate_up", "combine"};
  return (stage >= 0 && stage < MOE_STAGE_COUNT) ? names[stage] : "?";
}

int moe_workspace_size(const moe_desc *desc, size_t *bytes) {
  const int rc = check_desc(desc);
  if (rc) return rc;
  if (!bytes) return MOE_ERR_NULL;
  *bytes = layout_of(desc).total;
  return MOE_OK;
}

int moe_route(const moe_desc *d, const moe_weights *w, const void *x, int32_t *idx, float *g,
              float *gap, float *top_scores, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (!w || !w->w_router || !idx || !g || !ws || (!x && d->T > 0)) return MOE_ERR_NULL;
  if (!aligned16({x, ws}) || !weights_aligned(w)) return MOE_ERR_SHAPE;
  const Layout L = layout_of(d);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  RouterArgs a{};
  a.w_split = static_cast<char *>(ws) + L.wsplit;
  a.logits = reinterpret_cast<float *>(static_cast<char *>(ws) + L.logits);
  a.x = x;
  a.w = w->w_router;
  a.bias = w->bias;
  a.T = d->T;
  a.d = d->d_model;
  a.E = d->n_experts;
  a.K = d->top_k;
  a.mode = d->route_mode;
  a.renormalize = d->renormalize;
  a.routed_scale = d->routed_scale;
  a.idx = idx;
  a.g = g;
  a.gap = gap;
  a.top = top_scores;
  if (launch_router(a, d->act_dtype == MOE_BF16, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_quantile_balance(const moe_desc *d, const moe_weights *w, const void *x,
                         float *new_bias, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (d->route_mode != MOE_ROUTE_SIGMOID_BIAS) return MOE_ERR_MODE;
  if (d->top_k >= d->n_experts) return MOE_ERR_SHAPE;
  if (!w || !w->w_router || !new_bias || !ws || (!x && d->T > 0)) return MOE_ERR_NULL;
  if (!aligned16({x, ws}) || !weights_aligned(w)) return MOE_ERR_SHAPE;
  const Layout L = layout_of(d);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (d->T == 0) return MOE_OK;
  char *wsb = static_cast<char *>(ws);
  RouterArgs a{};
  a.w_split = wsb + L.wsplit;
  a.logits = reinterpret_cast<float *>(wsb + L.logits);
  a.x = x;
  a.w = w->w_router;
  a.bias = w->bias;
  a.T = d->T;
  a.d = d->d_model;
  a.E = d->n_experts;
  a.K = d->top_k;
  a.mode = d->route_mode;
  a.renormalize = d->renormalize;
  a.routed_scale = d->routed_scale;
  a.idx = reinterpret_cast<int32_t *>(wsb + L.idx);
  a.g = reinterpret_cast<float *>(wsb + L.g);
  a.gap = nullptr;
  a.top = reinterpret_cast<float *>(wsb + L.qb_top);
  if (launch_quantile_balance(a, d->act_dtype == MOE_BF16, reinterpret_cast<float *>(wsb + L.qb_diff),
                              reinterpret_cast<float *>(wsb + L.qb_q), new_bias,
                              static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_router_losses(const moe_desc *d, const moe_weights *w, const void *x,
                      const int32_t *counts, float alpha, float z_weight, float *losses, void *ws,
                      size_t ws_bytes, void *stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (!w || !w->w_router || !counts || !losses || !ws || (!x && d->T > 0)) return MOE_ERR_NULL;
  if (!aligned16({x, ws}) || !weights_aligned(w)) return MOE_ERR_SHAPE;
  if (!(alpha == alpha) || alpha > 3.4e38f || alpha < -3.4e38f || !(z_weight == z_weight) ||
      z_weight > 3.4e38f || z_weight < -3.4e38f)
    return MOE_ERR_MODE;
  const Layout L = layout_of(d);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (d->T == 0) return MOE_OK;
  char *wsb = static_cast<char *>(ws);
  RouterArgs a{};
  a.w_split = wsb + L.wsplit;
  a.logits = reinterpret_cast<float *>(wsb + L.logits);
  a.x = x;
  a.w = w->w_router;
  a.T = d->T;
  a.d = d->d_model;
  a.E = d->n_experts;
  a.K = d->top_k;
  if (launch_router_losses(a, d->act_dtype == MOE_BF16, counts, alpha, z_weight,
                           reinterpret_cast<float *>(wsb + L.loss), losses,
                           static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_dispatch(const moe_desc *d, const int32_t *idx, const float *g, const void *rows,
                 int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *sorted_token,
                 int32_t *inv, float *sorted_w, void *rows_sorted, void *ws, size_t ws_bytes,
                 void *stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (!counts || !offsets || !perm || !sorted_token || !inv || !ws) return MOE_ERR_NULL;
  if ((!idx && d->T > 0) || (sorted_w && !g) || (rows_sorted && !rows)) return MOE_ERR_NULL;
  if (!aligned16({rows, rows_sorted, ws})) return MOE_ERR_SHAPE;
  const Layout L = layout_of(d);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *wsb = static_cast<char *>(ws);
  const int64_t slots = d->T * d->top_k;
  int32_t *chunk = reinterpret_cast<int32_t *>(wsb + L.chunk);
  ScanArgs sa{};
  sa.chunk_hist = chunk;
  sa.chunk_base = chunk;
  sa.slots = slots;
  sa.E = d->n_experts;
  sa.counts = counts;
  sa.offsets = offsets;
  ScatterArgs sc{};
  sc.idx = idx;
  sc.g = g;
  sc.chunk_base = chunk;
  sc.slots = slots;
  sc.K = d->top_k;
  sc.E = d->n_experts;
  sc.perm = perm;
  sc.sorted_token = sorted_token;
  sc.inv = inv;
  sc.sorted_w = sorted_w;
  MOE_TRY(run_dispatch(sa, sc, s));
  if (rows_sorted) {
    const int64_t de = d->latent ? d->latent : d->d_model;
    const int64_t es = d->act_dtype == MOE_BF16 ? 2 : 4;
    MOE_TRY(launch_gather(rows, sorted_token, slots, de * es, rows_sorted, s));
  }
  return MOE_OK;
}

Tables tables_of(char *wsb, const Layout &L, const Plan &pl) {
  const int32_t *t1 = reinterpret_cast<int32_t *>(wsb + L.tiles);
  const int32_t *n1 = reinterpret_cast<int32_t *>(wsb + L.ntiles);
  if (pl.shared_table()) return {t1, n1, t1, n1};
  return {t1, n1, reinterpret_cast<int32_t *>(wsb + L.tiles2),
          reinterpret_cast<int32_t *>(wsb + L.ntiles2)};
}

int moe_expert_ffn(const moe_desc *d, const moe_weights *w, const void *rows,
                   const int32_t *row_index, const int32_t *offsets, const float *row_scale,
                   void *y_sorted, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if ((rc = check_expert_weights(d, w))) return rc;
  if (!offsets || !y_sorted || !ws || (!rows && d->T > 0)) return MOE_ERR_NULL;
  if (!aligned16({rows, y_sorted, ws}) || !weights_aligned(w)) return MOE_ERR_SHAPE;
  const Layout L = layout_of(d);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (d->T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *wsb = static_cast<char *>(ws);
  const Plan pl = plan_grouped(d);
  const Tables tb = tables_of(wsb, L, pl);
  MOE_TRY(launch_tiles(offsets, d->n_experts, pl.gu.bm(), const_cast<int32_t *>(tb.gu),
                       const_cast<int32_t *>(tb.gu_n), s));
  if (!pl.shared_table())
    MOE_TRY(launch_tiles(offsets, d->n_experts, pl.dn.bm(), const_cast<int32_t *>(tb.dn),
                         const_cast<int32_t *>(tb.dn_n), s));
  const Probe pr{nullptr, s};
  return expert_gemms(d, w, rows, row_index, tb, pl, row_scale, wsb + L.h, y_sorted, pr, s);
}

int moe_combine(const moe_desc *d, const moe_weights *w, const void *x, const void *y_sorted,
                const int32_t *inv, void *out, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if ((rc = check_combine_weights(d, w))) return rc;
  if (d->T > 0 && (!y_sorted || !inv || !out || (d->d_shared && !x))) return MOE_ERR_NULL;
  if (!ws) return MOE_ERR_NULL;
  if (!aligned16({x, y_sorted, out, ws}) || !weights_aligned(w)) return MOE_ERR_SHAPE;
  const Layout L = layout_of(d);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (d->T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Probe pr{nullptr, s};
  return shared_combine(d, w, x, y_sorted, inv, out, static_cast<char *>(ws), L, pr, s);
}

}  // extern "C"

namespace {

// Per-device address of `scratch` (set once per device, under the lock).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices];

int scratch_of(hipStream_t s, void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  if (s) {  // the stream's device must be the current one (whose copy is looked up)
    hipDevice_t sd = -1;
    if (hipStreamGetDevice(s, &sd) != hipSuccess) return MOE_ERR_HIP;
    if (sd != dev) return MOE_ERR_SCRATCH;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

int forward_impl(const moe_desc *d, const moe_weights *w, const void *x, void *out,
                 int32_t *counts, int32_t *n_near_ties, void *ws, size_t ws_bytes,
                 const moe_probe *probe, void *stream);

// A second stream per device (default priority) and three events, created on
// the first forward that overlaps there and kept until the process ends:
// the shared experts' first GEMM (and the latent down-projection) depend on x
// alone, so they run beside the routing, dispatch and routed GEMMs, which use
// few CUs at a time (router, dispatch) or leave CUs idle in their tails.
// The lock is held while a forward enqueues, so each event's record and the
// waits on it come from one call.
struct Side {
  hipStream_t s2 = nullptr;
  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
};
std::mutex g_side_mu;
Side g_side[kMaxDevices];

int side_of(hipStream_t s, Side **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  if (s) {
    hipDevice_t sd = -1;
    if (hipStreamGetDevice(s, &sd) != hipSuccess || sd != dev) return MOE_ERR_HIP;
  }
  Side &sd = g_side[dev];
  if (!sd.s2) {
    if (hipStreamCreateWithFlags(&sd.s2, hipStreamNonBlocking) != hipSuccess) return MOE_ERR_HIP;
    for (hipEvent_t &e : sd.ev)
      if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return MOE_ERR_HIP;
  }
  *out = &sd;
  return MOE_OK;
}

// Run the shared experts' first GEMM on the side stream: large bf16 layers
// whose shared GEMMs are separate launches, not under a timing probe.
bool overlap_shared(const moe_desc *d, bool merged, const moe_probe *probe) {
  return !probe && !merged && d->d_shared > 0 && d->act_dtype == MOE_BF16 && d->T >= 1024;
}

}  // namespace

extern "C" {

int moe_forward(const moe_desc *d, const moe_weights *w, const void *x, void *out,
                int32_t *counts, int32_t *n_near_ties, void *ws, size_t ws_bytes,
                const moe_probe *probe, void *stream) {
  return forward_impl(d, w, x, out, counts, n_near_ties, ws, ws_bytes, probe, stream);
}

int moe_forward_noalloc(const moe_desc *d, const moe_weights *w, const void *x, void *out,
                        int32_t *counts, int32_t *n_near_ties, void *stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (layout_of(d).total > MOE_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  if (!w || !w->w_router || (d->T > 0 && (!x || !out))) return MOE_ERR_NULL;
  if (!aligned16({x, out}) || !weights_aligned(w)) return MOE_ERR_SHAPE;
  void *ws = nullptr;
  if ((rc = scratch_of(static_cast<hipStream_t>(stream), &ws))) return rc;
  return forward_impl(d, w, x, out, counts, n_near_ties, ws, MOE_SCRATCH_BYTES, nullptr, stream);
}

}  // extern "C"

namespace {

int forward_impl(const moe_desc *d, const moe_weights *w, const void *x, void *out,
                 int32_t *counts, int32_t *n_near_ties, void *ws, size_t ws_bytes,
                 const moe_probe *probe, void *stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (!w || !w->w_router) return MOE_ERR_NULL;
  if ((rc = check_expert_weights(d, w)) || (rc = check_combine_weights(d, w))) return rc;
  if (d->latent && !w->w_lat_down) return MOE_ERR_NULL;
  if (!ws || (d->T > 0 && (!x || !out))) return MOE_ERR_NULL;
  if (!aligned16({x, out, ws}) || !weights_aligned(w)) return MOE_ERR_SHAPE;
  const Layout L = layout_of(d);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Probe pr{probe, s};
  char *wsb = static_cast<char *>(ws);
  const int64_t T = d->T, K = d->top_k, E = d->n_experts, rows = T * K;
  const int bf = d->act_dtype == MOE_BF16;
  int32_t *idx = reinterpret_cast<int32_t *>(wsb + L.idx);
  float *g = reinterpret_cast<float *>(wsb + L.g);
  float *gap = reinterpret_cast<float *>(wsb + L.gap);
  int32_t *cnt = counts ? counts : reinterpret_cast<int32_t *>(wsb + L.counts);
  int32_t *offsets = reinterpret_cast<int32_t *>(wsb + L.offsets);
  int32_t *chunk = reinterpret_cast<int32_t *>(wsb + L.chunk);
  int32_t *perm = reinterpret_cast<int32_t *>(wsb + L.perm);
  int32_t *stok = reinterpret_cast<int32_t *>(wsb + L.stok);
  int32_t *inv = reinterpret_cast<int32_t *>(wsb + L.inv);
  float *sw = reinterpret_cast<float *>(wsb + L.sw);
  const Plan pl = plan_grouped(d);
  const Tables tb = tables_of(wsb, L, pl);

  // 0. fork: the shared experts' first GEMM (latent: after the latent
  // down-projection, which the routed rows wait for) on the side stream
  const bool side = d->T > 0 && overlap_shared(d, pl.merged, probe);
  std::unique_lock<std::mutex> side_lock(g_side_mu, std::defer_lock);
  Side *sd = nullptr;
  if (side) {
    side_lock.lock();
    if ((rc = side_of(s, &sd))) return rc;
    MOE_TRY(hipEventRecord(sd->ev[0], s));
    MOE_TRY(hipStreamWaitEvent(sd->s2, sd->ev[0], 0));
    if (d->latent) {
      GemmArgs a{};
      a.a = x;
      a.lda = d->d_model;
      a.b0 = w->w_lat_down;
      a.ldb = d->d_model;
      a.K = d->d_model;
      a.N = d->latent;
      a.M = T;
      a.out = wsb + L.z;
      a.ldo = d->latent;
      MOE_TRY(launch_dense(a, EPI_STORE, bf, sd->s2));
      MOE_TRY(hipEventRecord(sd->ev[1], sd->s2));
    }
    if ((rc = shared_gate_up(d, w, x, wsb, L, Probe{nullptr, sd->s2}, sd->s2))) return rc;
    MOE_TRY(hipEventRecord(sd->ev[2], sd->s2));
  }

  // 1. router
  RouterArgs ra{};
  ra.x = x;
  ra.w = w->w_router;
  ra.w_split = wsb + L.wsplit;
  ra.logits = reinterpret_cast<float *>(wsb + L.logits);
  ra.bias = w->bias;
  ra.T = T;
  ra.d = d->d_model;
  ra.E = static_cast<int>(E);
  ra.K = static_cast<int>(K);
  ra.mode = d->route_mode;
  ra.renormalize = d->renormalize;
  ra.routed_scale = d->routed_scale;
  ra.idx = idx;
  ra.g = g;
  ra.gap = gap;
  pr.begin(MOE_STAGE_ROUTE);
  MOE_TRY(launch_router(ra, bf, s));
  pr.end(MOE_STAGE_ROUTE);

  // 2. dispatch (counts, offsets, tile table, stable positions)
  pr.begin(MOE_STAGE_DISPATCH);
  ScanArgs sa{};
  sa.chunk_hist = chunk;
  sa.chunk_base = chunk;
  sa.slots = rows;
  sa.E = static_cast<int>(E);
  sa.counts = cnt;
  sa.offsets = offsets;
  sa.bm = pl.gu.bm();
  sa.tiles = const_cast<int32_t *>(tb.gu);
  sa.n_tiles = const_cast<int32_t *>(tb.gu_n);
  if (!pl.shared_table()) {
    sa.bm2 = pl.dn.bm();
    sa.tiles2 = const_cast<int32_t *>(tb.dn);
    sa.n_tiles2 = const_cast<int32_t *>(tb.dn_n);
  }
  sa.gap = n_near_ties ? gap : nullptr;
  sa.T = T;
  sa.tie_eps = kTieEps;
  sa.n_near_ties = n_near_ties;
  ScatterArgs sc{};
  sc.idx = idx;
  sc.g = g;
  sc.chunk_base = chunk;
  sc.slots = rows;
  sc.K = static_cast<int>(K);
  sc.E = static_cast<int>(E);
  sc.perm = perm;
  sc.sorted_token = stok;
  sc.inv = inv;
  sc.sorted_w = sw;
  MOE_TRY(run_dispatch(sa, sc, s));
  pr.end(MOE_STAGE_DISPATCH);
  if (T == 0) return MOE_OK;

  // 3. latent down-projection (routed rows are z = x W_lat_down^T)
  const void *rsrc = x;
  if (d->latent && side) {
    MOE_TRY(hipStreamWaitEvent(s, sd->ev[1], 0));
    rsrc = wsb + L.z;
  } else if (d->latent) {
    GemmArgs a{};
    a.a = x;
    a.lda = d->d_model;
    a.b0 = w->w_lat_down;
    a.ldb = d->d_model;
    a.K = d->d_model;
    a.N = d->latent;
    a.M = T;
    a.out = wsb + L.z;
    a.ldo = d->latent;
    pr.begin(MOE_STAGE_LATENT_DOWN);
    for (int r = 0; r < pr.reps(MOE_STAGE_LATENT_DOWN); ++r)
      MOE_TRY(launch_dense(a, EPI_STORE, bf, s));
    pr.end(MOE_STAGE_LATENT_DOWN);
    rsrc = wsb + L.z;
  }

  // 4. grouped expert SwiGLU (gather fused into GEMM 1's A load), shared
  // experts, combine
  if (pl.merged) return merged_gemms(d, w, x, rsrc, stok, tb, pl, sw, inv, out, wsb, L, pr, s);
  if ((rc = expert_gemms(d, w, rsrc, stok, tb, pl, sw, wsb + L.h, wsb + L.y, pr, s)))
    return rc;
  if (side) MOE_TRY(hipStreamWaitEvent(s, sd->ev[2], 0));  // join
  return shared_combine(d, w, x, wsb + L.y, inv, out, wsb, L, pr, s, side);
}

}  // namespace

extern "C" {

int moe_backward_workspace_size(const moe_desc *desc, size_t *bytes) {
  const int rc = check_backward(desc);
  if (rc) return rc;
  if (!bytes) return MOE_ERR_NULL;
  *bytes = bwd_layout_of(desc).total;
  return MOE_OK;
}

int moe_backward(const moe_desc *d, const moe_weights *w, const void *x, const void *d_out,
                 void *d_x, const moe_grads *gr, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_backward(d);
  if (rc) return rc;
  if (!w || !w->w_router || !gr) return MOE_ERR_NULL;
  if ((rc = check_expert_weights(d, w)) || (rc = check_combine_weights(d, w))) return rc;
  if (d->latent && !w->w_lat_down) return MOE_ERR_NULL;
  if (!ws || (d->T > 0 && (!x || !d_out))) return MOE_ERR_NULL;
  if (!aligned16({x, d_out, d_x, ws, gr->w_router, gr->w_gate, gr->w_up, gr->w_down, gr->ws_gate,
                  gr->ws_up, gr->ws_down, gr->w_lat_down, gr->w_lat_up, gr->rms_gamma}) ||
      !weights_aligned(w))
    return MOE_ERR_SHAPE;
  const BwdLayout B = bwd_layout_of(d);
  if (ws_bytes < B.total) return MOE_ERR_WORKSPACE;
  if (d->T == 0) return MOE_OK;
  const Layout L = layout_of(d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *wsb = static_cast<char *>(ws);
  auto F = [&](size_t off) { return reinterpret_cast<float *>(wsb + off); };
  auto I = [&](size_t off) { return reinterpret_cast<int32_t *>(wsb + off); };
  const int64_t T = d->T, K = d->top_k, E = d->n_experts, rows = T * K;
  const int dm = d->d_model, f = d->d_ff, ds = d->d_shared, Lt = d->latent;
  const int de = Lt ? Lt : dm;  // routed width
  const int bf = d->act_dtype == MOE_BF16;
  const size_t es = bf ? 2 : 4;  // act element size
  int32_t *idx = I(L.idx), *counts = I(L.counts), *offsets = I(L.offsets);
  int32_t *stok = I(L.stok), *inv = I(L.inv);
  float *sw = F(L.sw);

  // 1. the forward's routing and dispatch (the selection defines the graph)
  RouterArgs ra{};
  ra.x = x;
  ra.w = w->w_router;
  ra.w_split = wsb + L.wsplit;
  ra.logits = F(L.logits);
  ra.bias = w->bias;
  ra.T = T;
  ra.d = dm;
  ra.E = static_cast<int>(E);
  ra.K = static_cast<int>(K);
  ra.mode = d->route_mode;
  ra.renormalize = d->renormalize;
  ra.routed_scale = d->routed_scale;
  ra.idx = idx;
  ra.g = F(L.g);
  ra.gap = F(L.gap);
  MOE_TRY(launch_router(ra, bf, s));
  ScanArgs sa{};
  sa.chunk_hist = I(L.chunk);
  sa.chunk_base = I(L.chunk);
  sa.slots = rows;
  sa.E = static_cast<int>(E);
  sa.counts = counts;
  sa.offsets = offsets;
  ScatterArgs sc{};
  sc.idx = idx;
  sc.g = ra.g;
  sc.chunk_base = I(L.chunk);
  sc.slots = rows;
  sc.K = static_cast<int>(K);
  sc.E = static_cast<int>(E);
  sc.perm = I(L.perm);
  sc.sorted_token = stok;
  sc.inv = inv;
  sc.sorted_w = sw;
  MOE_TRY(run_dispatch(sa, sc, s));
  // bf16: the pipelined kernel (two problems per launch where they pair up);
  // fp32: the generic kernel, 128 x 128 tiles, one problem per launch
  const int cfg = bf ? gemm2_pick(rows, E, de, f, 0, rows, f) : TILE_LARGE;
  const int bm = bf ? gemm2_bm(cfg) : tile_bm(TILE_LARGE);
  MOE_TRY(launch_tiles(offsets, static_cast<int>(E), bm, I(B.tiles), I(B.ntiles), s));
  const int64_t mt_bound = grouped_tile_bound(rows, E, bm);

  auto grouped = [&](const void *a, int64_t lda, const int32_t *a_rows, int64_t a_extent,
                     const void *b, int64_t ldb, int64_t b_stride, int Kd, int N, void *out,
                     int64_t ldo) {
    GemmArgs g{};
    g.a = a;
    g.lda = lda;
    g.a_rows = a_rows;
    g.a_extent = a_extent;
    g.b0 = b;
    g.ldb = ldb;
    g.b_stride = b_stride;
    g.K = Kd;
    g.N = N;
    g.M = rows;
    g.tiles = I(B.tiles);
    g.n_tiles = I(B.ntiles);
    g.max_mtiles = mt_bound;
    g.out = out;
    g.ldo = ldo;
    return g;
  };
  auto dense = [&](const void *a, int64_t lda, const void *b, int64_t ldb, int Kd, int N,
                   int64_t M, void *out, int64_t ldo) {
    GemmArgs g{};
    g.a = a;
    g.lda = lda;
    g.b0 = b;
    g.ldb = ldb;
    g.K = Kd;
    g.N = N;
    g.M = M;
    g.out = out;
    g.ldo = ldo;
    return g;
  };
  // 2. the products that read W_down, W_gate, W_up (and the shared FFN's and
  //    the latent projections) along their first dimension: bf16 layers
  //    read those weights in place, K-major on the pipelined kernel (the
  //    input gradient as two K segments, gate then up, which needs d_ff and
  //    d_shared to be multiples of 64); otherwise the active experts'
  //    weights are transposed first.
  const int64_t fe = static_cast<int64_t>(f) * de;
  auto kmajor = [&](GemmArgs g, const void *b, int64_t ldb, int64_t b_stride) {
    g.b0 = b;
    g.ldb = ldb;
    g.b_stride = b_stride;
    g.b_kmajor = 1;
    return g;
  };
  auto two_seg = [&](GemmArgs g, const char *a2, int64_t lda2, int K2, const void *b2,
                     int64_t ldb2, int64_t b2_stride) {
    g.a2 = a2;
    g.lda2 = lda2;
    g.K2 = K2;
    g.b2 = b2;
    g.ldb2 = ldb2;
    g.b2_stride = b2_stride;
    return g;
  };
  // dh = dy W_down per row (W_down [de, f]), shared dh = dy Ws_down ([d, ds])
  const GemmArgs gd_k = kmajor(grouped(nullptr, de, stok, T, nullptr, 0, 0, de, f, F(B.dhu), f),
                               w->w_down, f, fe);
  const GemmArgs sd_k = kmajor(dense(d_out, dm, nullptr, 0, dm, ds, T, F(B.dhu_s), ds),
                               w->ws_down, ds, 0);
  // dX = da W_gate + du W_up per row (W_gate, W_up [f, de]); shared alike
  const GemmArgs gx_k =
      two_seg(kmajor(grouped(wsb + B.dau, 2 * f, nullptr, rows, nullptr, 0, 0, f, de, F(B.dxs),
                             de),
                     w->w_gate, de, fe),
              wsb + B.dau + static_cast<size_t>(f) * es, 2 * f, f, w->w_up, de, fe);
  const GemmArgs sx_k =
      two_seg(kmajor(dense(wsb + B.dau_s, 2 * ds, nullptr, 0, ds, dm, T, F(B.dxsh), dm),
                     w->ws_gate, dm, 0),
              wsb + B.dau_s + static_cast<size_t>(ds) * es, 2 * ds, ds, w->ws_up, dm, 0);
  // latent: dR' = dy W_lat_up ([d, L]), dx_lat = dz W_lat_down ([L, d])
  const GemmArgs gp_k = kmajor(dense(d_out, dm, nullptr, 0, dm, Lt, T, F(B.dRp), Lt),
                               w->w_lat_up, Lt, 0);
  const GemmArgs gl_k = kmajor(dense(wsb + B.dz, Lt, nullptr, 0, Lt, dm, T, F(B.dxl), dm),
                               w->w_lat_down, dm, 0);
  const KmajorUse ku = kmajor_use(d);
  const bool km_dh = ku.dh, km_dx = ku.dx, km_lat = ku.lat;
  if (!km_dx) {
    MOE_TRY(launch_transpose(w->w_gate, E, f, de, counts, wsb + B.wguT, 2 * f, de * 2 * f, 0, bf, s));
    MOE_TRY(launch_transpose(w->w_up, E, f, de, counts, wsb + B.wguT, 2 * f, de * 2 * f, f, bf, s));
    if (ds) {
      MOE_TRY(launch_transpose(w->ws_gate, 1, ds, dm, nullptr, wsb + B.wsguT, 2 * ds, 0, 0, bf, s));
      MOE_TRY(launch_transpose(w->ws_up, 1, ds, dm, nullptr, wsb + B.wsguT, 2 * ds, 0, ds, bf, s));
    }
  }
  if (!km_dh) {
    MOE_TRY(launch_transpose(w->w_down, E, de, f, counts, wsb + B.wdT, de, f * de, 0, bf, s));
    if (ds)
      MOE_TRY(launch_transpose(w->ws_down, 1, dm, ds, nullptr, wsb + B.wsdT, dm, 0, 0, bf, s));
  }
  if (Lt && !km_lat) {
    MOE_TRY(launch_transpose(w->w_lat_up, 1, dm, Lt, nullptr, wsb + B.wluT, dm, 0, 0, bf, s));
    MOE_TRY(launch_transpose(w->w_lat_down, 1, Lt, dm, nullptr, wsb + B.wldT, Lt, 0, 0, bf, s));
  }

  auto gemm = [&](const GemmArgs &a, const GemmArgs *b, int c, int epi = EPI_STORE_F32) -> int {
    if (!bf) {  // generic kernel, one problem per launch
      if (launch_gemm(a, epi, TILE_LARGE, 0, s) != hipSuccess) return MOE_ERR_HIP;
      if (b && launch_gemm(*b, epi, TILE_LARGE, 0, s) != hipSuccess) return MOE_ERR_HIP;
      return MOE_OK;
    }
    if (!gemm2_applicable(a, epi) || (b && !gemm2_applicable(*b, epi))) return MOE_ERR_SHAPE;
    // K-major B: the 2x4-wavefront 256x256 tile (four B fragments per
    // wavefront instead of eight) loses less to the transposing reads
    if (a.b_kmajor && c == TILE2_256x256_TALLW) c = TILE2_256x256;
    return launch_gemm2(a, epi, c, s, b) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  };
  auto pick_dense = [&](int64_t M, int Kd, int N) { return gemm2_pick(M, 0, Kd, N, 0); };
  const int cfg_s = ds ? gemm2_pick(T, 0, dm, ds, 0, T, ds) : cfg;

  // routed input rows (x, or z = x W_lat_down^T as the forward computes it)
  const void *rin = x;
  if (Lt) {
    GemmArgs gz = dense(x, dm, w->w_lat_down, dm, dm, Lt, T, wsb + L.z, Lt);
    MOE_TRY(launch_dense(gz, EPI_STORE, bf, s));
    rin = wsb + L.z;
  }

  // 3. pre-activations a, u (fp32), routed and shared: as one gate/up tile
  //    (the forward's, both halves stored in fp32) on the persistent kernel
  //    where it takes the launch, else as two problems of one launch
  auto gate_up_f32 = [&](GemmArgs ga, GemmArgs gu, int c) -> int {
    GemmArgs g = ga;
    g.b1 = gu.b0;
    g.out2 = gu.out;
    if (bf && gemm2_applicable(g, EPI_GLU_F32) && gemm2_persistent(g, EPI_GLU_F32, c))
      return launch_gemm2(g, EPI_GLU_F32, c, s) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
    return gemm(ga, &gu, c);
  };
  {
    const GemmArgs ga = grouped(rin, de, stok, T, w->w_gate, de, static_cast<int64_t>(f) * de, de,
                                f, F(B.apre), f);
    const GemmArgs gu = grouped(rin, de, stok, T, w->w_up, de, static_cast<int64_t>(f) * de, de,
                                f, F(B.upre), f);
    if ((rc = gate_up_f32(ga, gu, cfg))) return rc;
    if (ds) {
      const GemmArgs sa2 = dense(x, dm, w->ws_gate, dm, dm, ds, T, F(B.apre_s), ds);
      const GemmArgs su = dense(x, dm, w->ws_up, dm, dm, ds, T, F(B.upre_s), ds);
      if ((rc = gate_up_f32(sa2, su, cfg_s))) return rc;
    }
  }

  // routed output gradient per token: d_out, or (latent) the RMSNorm
  // backward of W_lat_up^T d_out on the recomputed routed sum
  const void *rdy = d_out;
  if (Lt) {
    MOE_TRY(launch_bwd_rows(F(B.apre), F(B.upre), nullptr, nullptr, rows, f, wsb + B.h, nullptr,
                            nullptr, bf, s));
    GemmArgs gy = grouped(wsb + B.h, f, nullptr, rows, w->w_down, f,
                          static_cast<int64_t>(Lt) * f, f, Lt, F(B.yf), Lt);
    gy.row_scale = sw;
    gy.out_f32 = 1;
    if ((rc = gemm(gy, nullptr, cfg, EPI_SCALE))) return rc;
    MOE_TRY(launch_latent_fwd(F(B.yf), inv, T, static_cast<int>(K), Lt, d->has_rmsnorm,
                              d->rms_eps, w->rms_gamma, F(B.R), F(B.rinv), wsb + B.Rp, bf, s));
    const GemmArgs gp =
        km_lat ? gp_k : dense(d_out, dm, wsb + B.wluT, dm, dm, Lt, T, F(B.dRp), Lt);
    if ((rc = gemm(gp, nullptr, pick_dense(T, dm, Lt)))) return rc;
    MOE_TRY(launch_latent_bwd(F(B.dRp), F(B.R), F(B.rinv), w->rms_gamma, T, Lt,
                              d->has_rmsnorm, wsb + B.dR, bf, s));
    rdy = wsb + B.dR;
  }

  // 4. W_down^T dy per sorted row (unscaled) and per token for the shared FFN
  {
    GemmArgs gd = km_dh ? gd_k : grouped(nullptr, de, stok, T, wsb + B.wdT, de, fe, de, f,
                                         F(B.dhu), f);
    gd.a = rdy;
    if (ds) {
      const GemmArgs sd =
          km_dh ? sd_k : dense(d_out, dm, wsb + B.wsdT, dm, dm, ds, T, F(B.dhu_s), ds);
      if ((rc = gemm(gd, &sd, cfg))) return rc;
    } else if ((rc = gemm(gd, nullptr, cfg))) {
      return rc;
    }
  }
  // 5. h, [da | du], dg per row; the router's logit gradients
  MOE_TRY(launch_bwd_rows(F(B.apre), F(B.upre), F(B.dhu), sw, rows, f, wsb + B.h, wsb + B.dau,
                          F(B.dg), bf, s));
  if (ds)
    MOE_TRY(launch_bwd_rows(F(B.apre_s), F(B.upre_s), F(B.dhu_s), nullptr, T, ds, wsb + B.h_s,
                            wsb + B.dau_s, nullptr, bf, s));
  MOE_TRY(launch_router_backward(ra, bf, inv, F(B.dg), F(B.dr), s));

  // 6. input gradient: [da | du] [W_gate^T | W_up^T]^T per row (to x, or to z
  //    and through W_lat_down), shared, router
  const bool need_dz = d_x || (Lt && gr->w_lat_down);
  if (need_dz) {
    const GemmArgs gx = km_dx ? gx_k
                              : grouped(wsb + B.dau, 2 * f, nullptr, rows, wsb + B.wguT, 2 * f,
                                        static_cast<int64_t>(de) * 2 * f, 2 * f, de, F(B.dxs), de);
    if (ds) {
      const GemmArgs sx = km_dx ? sx_k
                                : dense(wsb + B.dau_s, 2 * ds, wsb + B.wsguT, 2 * ds, 2 * ds, dm,
                                        T, F(B.dxsh), dm);
      if ((rc = gemm(gx, &sx, cfg))) return rc;
    } else if ((rc = gemm(gx, nullptr, cfg))) {
      return rc;
    }
  }
  if (Lt && need_dz) {  // dz = sum_k dX rows (bf16), dx_lat = dz W_lat_down
    MOE_TRY(launch_bwd_dx(F(B.dxs), nullptr, nullptr, inv, idx, nullptr, nullptr, T,
                          static_cast<int>(K), Lt, wsb + B.dz, bf, s));
    if (d_x) {
      const GemmArgs gl =
          km_lat ? gl_k : dense(wsb + B.dz, Lt, wsb + B.wldT, Lt, Lt, dm, T, F(B.dxl), dm);
      if ((rc = gemm(gl, nullptr, pick_dense(T, Lt, dm)))) return rc;
    }
  }
  if (d_x)
    MOE_TRY(launch_bwd_dx(Lt ? nullptr : F(B.dxs), ds ? F(B.dxsh) : nullptr,
                          Lt ? F(B.dxl) : nullptr, inv, idx, F(B.dr), w->w_router, T,
                          static_cast<int>(K), dm, d_x, bf, s));

  // 7. weight gradients
  if (gr->w_router)
    MOE_TRY(launch_bwd_dwr(F(B.dr), stok, offsets, x, static_cast<int>(E), dm, F(B.dwr_part),
                           gr->w_router, bf, s));
  if (Lt && d->has_rmsnorm && gr->rms_gamma)
    MOE_TRY(launch_colsum(F(B.dRp), F(B.R), F(B.rinv), T, Lt, F(B.gpart), gr->rms_gamma, s));
  const bool want_e = gr->w_gate || gr->w_up || gr->w_down;
  const bool want_s = ds && (gr->ws_gate || gr->ws_up || gr->ws_down);
  const bool want_l = Lt && (gr->w_lat_up || gr->w_lat_down);
  const int cfg_k =
      bf ? gemm2_pick(E * (f > de ? f : de), 0, rows / E + 64, f < de ? f : de, 0) : TILE_LARGE;
  const int bm_k = bf ? gemm2_bm(cfg_k) : tile_bm(TILE_LARGE);
  if (want_e) {
    MOE_TRY(launch_kgroup(counts, static_cast<int>(E), f, de, bm_k, I(B.poff),
                          I(B.kt1), I(B.kn1), I(B.kt2), I(B.kn2), s));
    const int G = static_cast<int>(E);
    const int32_t *po = I(B.poff);
    const int64_t RP = B.RP;
    MOE_TRY(launch_cols(rin, de, stok, nullptr, rows, de, offsets, po, G, RP, wsb + B.xsT, RP, bf, s));
    MOE_TRY(launch_cols(rdy, de, stok, sw, rows, de, offsets, po, G, RP, wsb + B.dysT, RP, bf, s));
    MOE_TRY(launch_cols(wsb + B.dau, 2 * f, nullptr, nullptr, rows, f, offsets, po, G, RP,
                        wsb + B.daT, RP, bf, s));
    MOE_TRY(launch_cols(wsb + B.dau + static_cast<size_t>(f) * es, 2 * f, nullptr, nullptr, rows,
                        f, offsets, po, G, RP, wsb + B.duT, RP, bf, s));
    MOE_TRY(launch_cols(wsb + B.h, f, nullptr, nullptr, rows, f, offsets, po, G, RP, wsb + B.hT,
                        RP, bf, s));
    auto kgrouped = [&](const void *a, int64_t M, const void *b, int N, int32_t *tab,
                        int32_t *ntab, void *out) {
      GemmArgs g{};
      g.a = a;
      g.lda = B.RP;
      g.a_extent = M;
      g.b0 = b;
      g.ldb = B.RP;
      g.K = 64;
      g.N = N;
      g.tiles = tab;
      g.n_tiles = ntab;
      g.max_mtiles = E * ((M + bm_k - 1) / bm_k);
      g.k_offsets = I(B.poff);
      g.out = out;
      g.ldo = N;
      g.out_stride = M * N;
      return g;
    };
    if (gr->w_gate || gr->w_up) {
      const GemmArgs kg = kgrouped(wsb + B.daT, f, wsb + B.xsT, de, I(B.kt1), I(B.kn1),
                                   gr->w_gate ? static_cast<void *>(gr->w_gate) : nullptr);
      const GemmArgs ku = kgrouped(wsb + B.duT, f, wsb + B.xsT, de, I(B.kt1), I(B.kn1),
                                   gr->w_up ? static_cast<void *>(gr->w_up) : nullptr);
      if (gr->w_gate && gr->w_up) {
        if ((rc = gemm(kg, &ku, cfg_k))) return rc;
      } else if ((rc = gemm(gr->w_gate ? kg : ku, nullptr, cfg_k))) {
        return rc;
      }
    }
    if (gr->w_down) {
      const GemmArgs kd = kgrouped(wsb + B.dysT, de, wsb + B.hT, f, I(B.kt2), I(B.kn2),
                                   gr->w_down);
      if ((rc = gemm(kd, nullptr, cfg_k))) return rc;
    }
  }
  const int64_t TP = B.TP;
  const int TPk = static_cast<int>(TP);
  if (want_s || want_l) {
    MOE_TRY(launch_cols(x, dm, nullptr, nullptr, T, dm, nullptr, nullptr, 0, TP, wsb + B.xT, TP, bf, s));
    MOE_TRY(launch_cols(d_out, dm, nullptr, nullptr, T, dm, nullptr, nullptr, 0, TP, wsb + B.dyT,
                        TP, bf, s));
  }
  if (want_s) {
    MOE_TRY(launch_cols(wsb + B.dau_s, 2 * ds, nullptr, nullptr, T, ds, nullptr, nullptr, 0, TP,
                        wsb + B.dashT, TP, bf, s));
    MOE_TRY(launch_cols(wsb + B.dau_s + static_cast<size_t>(ds) * es, 2 * ds, nullptr, nullptr, T,
                        ds, nullptr, nullptr, 0, TP, wsb + B.dushT, TP, bf, s));
    MOE_TRY(launch_cols(wsb + B.h_s, ds, nullptr, nullptr, T, ds, nullptr, nullptr, 0, TP,
                        wsb + B.hshT, TP, bf, s));
    const int cfg_w = gemm2_pick(ds, 0, TPk, dm, 0, ds, dm);
    if (gr->ws_gate) {
      const GemmArgs g1 = dense(wsb + B.dashT, TP, wsb + B.xT, TP, TPk, dm, ds, gr->ws_gate, dm);
      if ((rc = gemm(g1, nullptr, cfg_w))) return rc;
    }
    if (gr->ws_up) {
      const GemmArgs g2 = dense(wsb + B.dushT, TP, wsb + B.xT, TP, TPk, dm, ds, gr->ws_up, dm);
      if ((rc = gemm(g2, nullptr, cfg_w))) return rc;
    }
    if (gr->ws_down) {
      const GemmArgs g3 = dense(wsb + B.dyT, TP, wsb + B.hshT, TP, TPk, ds, dm, gr->ws_down, ds);
      if ((rc = gemm(g3, nullptr, pick_dense(dm, TPk, ds)))) return rc;
    }
  }
  if (want_l) {
    if (gr->w_lat_up) {  // dW_lat_up = dy^T R' (d x L)
      MOE_TRY(launch_cols(wsb + B.Rp, Lt, nullptr, nullptr, T, Lt, nullptr, nullptr, 0, TP,
                          wsb + B.RpT, TP, bf, s));
      const GemmArgs gu = dense(wsb + B.dyT, TP, wsb + B.RpT, TP, TPk, Lt, dm, gr->w_lat_up, Lt);
      if ((rc = gemm(gu, nullptr, pick_dense(dm, TPk, Lt)))) return rc;
    }
    if (gr->w_lat_down) {  // dW_lat_down = dz^T x (L x d)
      MOE_TRY(launch_cols(wsb + B.dz, Lt, nullptr, nullptr, T, Lt, nullptr, nullptr, 0, TP,
                          wsb + B.dzT, TP, bf, s));
      const GemmArgs gd = dense(wsb + B.dzT, TP, wsb + B.xT, TP, TPk, dm, Lt, gr->w_lat_down, dm);
      if ((rc = gemm(gd, nullptr, pick_dense(Lt, TPk, dm)))) return rc;
    }
  }
  return MOE_OK;
}

int moe_plan(const moe_desc *d, moe_plan_info *info) {
  const int rc = check_desc(d);
  if (rc) return rc;
  if (!info) return MOE_ERR_NULL;
  const Plan pl = plan_grouped(d);
  RouterArgs ra{};
  ra.T = d->T;
  ra.d = d->d_model;
  ra.E = d->n_experts;
  *info = moe_plan_info{};
  info->merged_shared = pl.merged ? 1 : 0;
  info->gate_up_pipelined = pl.gu.v2;
  info->gate_up_tile_m = pl.gu.bm();
  info->gate_up_tile_n = pl.gu.v2 ? gemm2_bn(pl.gu.cfg) : tile_bn(pl.gu.cfg);
  info->down_pipelined = pl.dn.v2;
  info->down_tile_m = pl.dn.bm();
  info->down_tile_n = pl.dn.v2 ? gemm2_bn(pl.dn.cfg) : tile_bn(pl.dn.cfg);
  info->router_per_token = router_valu(ra) ? 1 : 0;
  info->dispatch_one_workgroup = dispatch_fused_ok(d->T * d->top_k, d->n_experts) ? 1 : 0;
  const KmajorUse ku = kmajor_use(d);
  info->backward_in_place = (ku.dh ? 1 : 0) | (ku.dx ? 2 : 0) | (ku.lat ? 4 : 0);
  // the grouped launches as expert_gemms makes them (a second, dense problem
  // when the shared experts are merged in)
  if (pl.gu.v2 && pl.dn.v2) {
    const int64_t rows_n = d->T * d->top_k;
    const int de = d->latent ? d->latent : d->d_model;
    static const int32_t kTable = 0;  // (only its presence matters here)
    GemmArgs a{}, b{}, sec{};
    a.tiles = b.tiles = &kTable;
    a.K = de;
    a.N = d->d_ff;
    a.ldo = d->d_ff;
    a.max_mtiles = grouped_tile_bound(rows_n, d->n_experts, pl.gu.bm());
    b.K = d->d_ff;
    b.N = b.ldo = de;
    b.max_mtiles = grouped_tile_bound(rows_n, d->n_experts, pl.dn.bm());
    sec.N = pl.merged ? 1 : 0;
    info->persistent = (gemm2_persistent(a, EPI_SWIGLU, pl.gu.cfg, &sec) ? 1 : 0) |
                       (gemm2_persistent(b, EPI_SCALE, pl.dn.cfg, &sec) ? 2 : 0);
  }
  return MOE_OK;
}

int moe_balance_bias(int32_t n_experts, int32_t top_k, int64_t n_tokens, const int32_t *counts,
                     float alpha, float *bias, void *stream) {
  if (n_experts < 1 || n_experts > 1024 || top_k < 1 || top_k > n_experts || n_tokens < 0 ||
      n_tokens * static_cast<int64_t>(top_k) > 0x7FFFFFFF)
    return MOE_ERR_SHAPE;
  if (!counts || !bias) return MOE_ERR_NULL;
  if (!(alpha == alpha) || alpha > 3.4e38f || alpha < -3.4e38f) return MOE_ERR_MODE;
  if (n_tokens == 0) return MOE_OK;
  MOE_TRY(launch_balance(n_experts, n_tokens * top_k, counts, alpha, bias,
                         static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

int moe_peak(int32_t mode, int32_t threads, int32_t groups, int32_t iters, int64_t *clk,
             uint32_t *sink, void *stream) {
  if (mode < 0 || mode > 10 || (threads != 256 && threads != 512) || groups < 1 ||
      groups > (1 << 20) || iters < 1)
    return MOE_ERR_SHAPE;
  if (!clk || !sink) return MOE_ERR_NULL;
  MOE_TRY(launch_peak(mode, threads, groups, iters, clk, sink, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

}  // extern "C"
