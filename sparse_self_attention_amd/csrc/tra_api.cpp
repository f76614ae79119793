// Host side of the C ABI declared in include/tra.h: validation, the radius
// table, plan ownership and kernel sequencing.  Every step of the path itself
// runs in the kernels of tra_kernels.hip.
#include "tra.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "tra_internal.h"

#include <rocprofiler-sdk-roctx/roctx.h>

namespace {

thread_local std::string g_last_error;

tra_status fail(tra_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

// Fault injection for tests of the error paths.  TRA_FAULT=alloc[:n] makes the
// n-th device or pinned-host allocation (default the first) of an API call
// fail as if the runtime were out of memory; TRA_FAULT=launch[:n] makes the
// n-th kernel launch fail.  Read at the start of every call that allocates or
// launches; unset (the normal case) it costs one getenv per call.
enum { FAULT_NONE = 0, FAULT_ALLOC = 1, FAULT_LAUNCH = 2 };
struct FaultState {
  int kind = FAULT_NONE, at = 0, count = 0;
};
thread_local FaultState g_fault;

// A named range on the profiler's marker timeline (rocprofv3 --marker-trace)
// for the scope's host-side work, kernel launches included.
struct Range {
  explicit Range(const char* name) { roctxRangePushA(name); }
  ~Range() { roctxRangePop(); }
  Range(const Range&) = delete;
  Range& operator=(const Range&) = delete;
};

void fault_arm() {
  g_fault = FaultState{};
  const char* f = std::getenv("TRA_FAULT");
  if (!f || !*f) return;
  int kind = FAULT_NONE;
  const char* rest = f;
  if (std::strncmp(f, "alloc", 5) == 0) {
    kind = FAULT_ALLOC;
    rest = f + 5;
  } else if (std::strncmp(f, "launch", 6) == 0) {
    kind = FAULT_LAUNCH;
    rest = f + 6;
  } else {
    return;
  }
  int at = 1;
  if (*rest == ':') at = std::atoi(rest + 1);
  else if (*rest) return;
  if (at < 1) return;
  g_fault.kind = kind;
  g_fault.at = at;
}

bool fault_hit(int kind) { return g_fault.kind == kind && ++g_fault.count == g_fault.at; }

hipError_t dev_alloc(void** p, size_t bytes) {
  *p = nullptr;
  if (fault_hit(FAULT_ALLOC)) return hipErrorOutOfMemory;
  return hipMalloc(p, bytes);
}

template <typename T>
hipError_t dev_alloc(T** p, size_t bytes) {
  void* v = nullptr;
  const hipError_t e = dev_alloc(&v, bytes);
  *p = static_cast<T*>(v);
  return e;
}

template <typename T>
hipError_t host_alloc(T** p, size_t bytes) {
  *p = nullptr;
  if (fault_hit(FAULT_ALLOC)) return hipErrorOutOfMemory;
  void* v = nullptr;
  const hipError_t e = hipHostMalloc(&v, bytes);
  *p = static_cast<T*>(v);
  return e;
}

// True when fault injection refuses the next kernel launch (which then does
// not happen).
bool launch_refused() { return fault_hit(FAULT_LAUNCH); }

#define TRA_HIP(call)                                                                    \
  do {                                                                                   \
    hipError_t e_ = (call);                                                              \
    if (e_ != hipSuccess) {                                                              \
      if (e_ == hipErrorOutOfMemory)                                                     \
        return fail(TRA_ERR_OOM, std::string(#call) + ": " + hipGetErrorString(e_));     \
      return fail(TRA_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_));       \
    }                                                                                    \
  } while (0)

// A kernel launch through one of the tra::launch_* wrappers.
#define TRA_LAUNCH(call)                                                                  \
  do {                                                                                   \
    if (launch_refused()) return fail(TRA_ERR_HIP, std::string("injected launch failure: ") + #call); \
    TRA_HIP(call);                                                                       \
  } while (0)

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// Level range and radius table, fp64 on the host.
struct Table {
  int k_lo = 0, k_hi = 0, n_levels = 0;
  std::vector<double> r0sq;     // per level row
  std::vector<int32_t> r2;      // n_levels x T, -1 = inactive frame
  std::vector<int32_t> dmax;    // largest active delta per row
  std::vector<int32_t> r2c;     // compact: active entries of each row, row r at r2off[r]
  std::vector<int32_t> r2off;
};

tra_status check_shape(const tra_shape* s) {
  if (!s) return fail(TRA_ERR_INVALID_ARG, "shape is NULL");
  if (s->B < 1 || s->heads < 1 || s->T < 1 || s->H < 1 || s->W < 1)
    return fail(TRA_ERR_SHAPE, "B, heads, T, H and W must be >= 1");
  if (s->H > 32767 || s->W > 32767 || s->T > 32767)
    return fail(TRA_ERR_SHAPE, "T, H and W must be <= 32767");
  const int64_t N = static_cast<int64_t>(s->T) * s->H * s->W;
  if (static_cast<int64_t>(s->B) * s->heads * N >= (int64_t(1) << 31))
    return fail(TRA_ERR_SHAPE, "B*heads*T*H*W must be below 2^31");
  if (s->dtype != TRA_F32 && s->dtype != TRA_BF16) return fail(TRA_ERR_DTYPE, "dtype must be TRA_F32 or TRA_BF16");
  if (s->head_dim != 64 && s->head_dim != 128) return fail(TRA_ERR_DTYPE, "head_dim must be 64 or 128");
  return TRA_OK;
}

tra_status check_params(const tra_shape* s, const tra_params* p, Table* tab) {
  if (!p) return fail(TRA_ERR_INVALID_ARG, "params is NULL");
  if (!std::isfinite(p->a) || !std::isfinite(p->c)) return fail(TRA_ERR_INVALID_ARG, "a and c must be finite");
  if (!(p->budget_min > 0.0) || !std::isfinite(p->budget_max) || !(p->budget_max >= p->budget_min))
    return fail(TRA_ERR_INVALID_ARG, "need 0 < budget_min <= budget_max < inf");
  if (!(p->decay > 0.0 && p->decay <= 1.0)) return fail(TRA_ERR_INVALID_ARG, "decay must lie in (0, 1]");
  if (p->levels_per_nat < 1 || p->levels_per_nat > 1024)
    return fail(TRA_ERR_INVALID_ARG, "levels_per_nat must lie in [1, 1024]");
  if (p->pool_h < 1 || p->pool_w < 1) return fail(TRA_ERR_INVALID_ARG, "pool_h and pool_w must be >= 1");
  if (p->tile_h != 8 || p->tile_w != 8)
    return fail(TRA_ERR_INVALID_ARG, "the device kernels use 8x8 tiles (tile_h = tile_w = 8)");
  if (s->dtype == TRA_BF16 &&
      static_cast<int64_t>(s->T) * s->H * s->W * s->head_dim * 2 >= (int64_t(1) << 31))
    return fail(TRA_ERR_SHAPE, "bf16 attention needs T*H*W*head_dim*2 (bytes of one head) below 2^31");
  if (!std::isfinite(p->radius_override) || p->radius_override >= 32768.0)
    return fail(TRA_ERR_INVALID_ARG, "radius_override must be finite and below 32768");
  if (p->generator < TRA_GEN_ENTROPY_DISK || p->generator > TRA_GEN_WINDOW_1D)
    return fail(TRA_ERR_INVALID_ARG, "unknown generator");
  if (p->generator == TRA_GEN_WINDOW_1D) {
    if ((s->W + p->tile_w - 1) / p->tile_w > 64)
      return fail(TRA_ERR_SHAPE, "the 1-D window generator builds its tile lists for at most 64 tile columns");
    if (p->vote_threshold > 1) return fail(TRA_ERR_INVALID_ARG, "the 1-D window generator takes vote_threshold 1");
  }
  if (p->vote_threshold < 1 || p->vote_threshold > p->tile_h * p->tile_w * p->tile_h * p->tile_w)
    return fail(TRA_ERR_INVALID_ARG, "vote_threshold must lie in [1, (tile_h*tile_w)^2]");
  if (p->block_mask != 0 && p->block_mask != 1) return fail(TRA_ERR_INVALID_ARG, "block_mask must be 0 or 1");
  if (p->regroup != 0 && p->regroup != 1) return fail(TRA_ERR_INVALID_ARG, "regroup must be 0 or 1");
  if (p->regroup && s->dtype != TRA_BF16)
    return fail(TRA_ERR_INVALID_ARG, "regroup is a layout of the bf16 attention kernel (dtype TRA_BF16)");
  // Block-only masks and vote-filtered lists are defined per query tile; a
  // regrouped wave holds queries of all four tiles of its group.
  if (p->regroup && (p->block_mask || p->vote_threshold > 1))
    return fail(TRA_ERR_INVALID_ARG, "regroup takes the exact mask with vote_threshold 1");
  if (p->group_rows != 0 && p->group_rows != 2 && p->group_rows != 3)
    return fail(TRA_ERR_INVALID_ARG, "group_rows must be 0 (automatic), 2 or 3");
  if (p->regroup && p->group_rows == 3)
    return fail(TRA_ERR_INVALID_ARG, "regroup orders the queries of 2 x 2 groups (group_rows 0 or 2)");
  if ((p->generator == TRA_GEN_MANHATTAN || p->generator == TRA_GEN_RADIAL) && !(p->radius_override >= 0.0))
    return fail(TRA_ERR_INVALID_ARG, "the Manhattan and Radial generators take their radius from radius_override (>= 0)");
  const int T = s->T;
  const double phi = p->decay;
  Table t;
  if (p->radius_override >= 0.0) {
    t.k_lo = -1;
    t.k_hi = -1;
    t.n_levels = 1;
    t.r0sq.push_back(p->radius_override * p->radius_override);
  } else {
    const double q = p->levels_per_nat;
    const double klo = std::ceil(q * std::log(p->budget_min));
    const double khi = std::floor(q * std::log(p->budget_max));
    if (!(klo <= khi)) return fail(TRA_ERR_INVALID_ARG, "budget range holds no quantisation level");
    if (khi - klo + 1 > 4096) return fail(TRA_ERR_INVALID_ARG, "more than 4096 budget levels");
    if (std::fabs(klo) > 30000 || std::fabs(khi) > 30000)
      return fail(TRA_ERR_INVALID_ARG, "budget levels do not fit int16");
    t.k_lo = static_cast<int>(klo);
    t.k_hi = static_cast<int>(khi);
    t.n_levels = t.k_hi - t.k_lo + 1;
    // S = sum over delta in [-(T-1), T-1] of phi^(2|delta|): every frame's disk
    // shares the budget, with area shrinking by phi^2 per frame of distance.
    double S = 0.0;
    for (int dl = -(T - 1); dl <= T - 1; ++dl) S += std::pow(phi, 2.0 * std::abs(dl));
    for (int k = t.k_lo; k <= t.k_hi; ++k) t.r0sq.push_back(std::exp(k / q) / (M_PI * S));
  }
  if (p->generator != TRA_GEN_WINDOW_1D && t.r0sq.back() >= 1073741824.0)
    return fail(TRA_ERR_INVALID_ARG, "radius^2 must stay below 2^30");
  // 1-D window half-widths: rho = floor((B - 1)/2) for budget B = exp(k/q), so
  // that the window of 2 rho + 1 tokens holds the budget (floor(r) under
  // radius_override).
  std::vector<int32_t> rho(t.n_levels, 0);
  if (p->generator == TRA_GEN_WINDOW_1D) {
    for (int r = 0; r < t.n_levels; ++r) {
      const double x = p->radius_override >= 0.0
                           ? std::floor(p->radius_override)
                           : std::floor((std::exp((t.k_lo + r) / static_cast<double>(p->levels_per_nat)) - 1.0) / 2.0);
      if (!(x < 16777216.0)) return fail(TRA_ERR_INVALID_ARG, "1-D window half-width must stay below 2^24");
      rho[r] = static_cast<int32_t>(x);
    }
  }
  const int64_t HW = static_cast<int64_t>(s->H) * s->W;
  if (static_cast<int64_t>(t.n_levels) * T > (int64_t(1) << 22))
    return fail(TRA_ERR_INVALID_ARG, "radius table too large");
  t.r2.resize(static_cast<size_t>(t.n_levels) * T);
  t.dmax.resize(t.n_levels);
  for (int r = 0; r < t.n_levels; ++r) {
    int dm = 0;
    for (int dl = 0; dl < T; ++dl) {
      int32_t v;
      if (p->generator == TRA_GEN_WINDOW_1D) {
        // The same rho in every column; frames beyond reach are marked by dmax
        // (the nearest tokens of frames dl apart are dl*H*W - (H*W - 1) apart).
        v = rho[r];
        if (dl * HW - (HW - 1) <= rho[r]) dm = dl;
        t.r2[static_cast<size_t>(r) * T + dl] = v;
        continue;
      }
      if (p->generator == TRA_GEN_MANHATTAN) {
        // L1 ball |dt| + |dh| + |dw| <= R: frame dl holds the 2D L1 disk of radius R - dl.
        v = static_cast<int32_t>(std::floor(p->radius_override)) - dl;
        if (v < 0) v = -1;
      } else {
        double x;
        if (p->generator == TRA_GEN_RADIAL) {
          // Octave band b of dl (0 | 1 | 2-3 | 4-7 | ...): the disk area halves per band.
          int band = 0;
          for (int u = dl; u > 0; u >>= 1) ++band;
          x = std::ldexp(t.r0sq[r], -band);
        } else {
          x = t.r0sq[r] * std::pow(phi, 2.0 * dl);
        }
        v = static_cast<int32_t>(std::floor(x));
        if (dl > 0 && v < 1) v = -1;
      }
      if (v >= 0) dm = dl;
      t.r2[static_cast<size_t>(r) * T + dl] = v;
    }
    t.dmax[r] = dm;
  }
  t.r2off.resize(t.n_levels);
  for (int r = 0; r < t.n_levels; ++r) {
    t.r2off[r] = static_cast<int32_t>(t.r2c.size());
    for (int dl = 0; dl <= t.dmax[r]; ++dl) t.r2c.push_back(t.r2[static_cast<size_t>(r) * T + dl]);
  }
  if ((2 * static_cast<size_t>(t.n_levels) + t.r2c.size()) * sizeof(int32_t) > 65536)
    return fail(TRA_ERR_INVALID_ARG, "radius table too large for the tile-list kernel's LDS");
  if (s->dtype == TRA_BF16 && tra::attention_lds_bytes(s->head_dim, static_cast<int>(t.r2c.size())) > 163840)
    return fail(TRA_ERR_INVALID_ARG, "radius table too large for the attention kernel's LDS");
  if (tab) *tab = std::move(t);
  return TRA_OK;
}

size_t dtype_size(int dtype) { return dtype == TRA_BF16 ? 2 : 4; }

int metric_of(const tra_params& p) {
  if (p.generator == TRA_GEN_MANHATTAN) return tra::METRIC_L1;
  if (p.generator == TRA_GEN_WINDOW_1D) return tra::METRIC_WINDOW;
  return tra::METRIC_L2;
}

}  // namespace

struct tra_plan {
  tra_shape shape;
  tra_params params;
  Table table;
  tra::Grid pool, tiles;
  int BH = 0;
  int64_t N = 0, n_queries = 0, n_rows = 0;
  int row_base = 0;
  int device = 0;
  // device buffers
  void* kbar = nullptr;
  float* H = nullptr;
  int16_t* lv = nullptr;
  int32_t* r2 = nullptr;
  int32_t* dmax = nullptr;
  int32_t* r2c = nullptr;
  int32_t* r2off = nullptr;
  float* pool_w = nullptr;
  int32_t* counts = nullptr;
  int32_t* row_ptr = nullptr;
  int32_t* col_idx = nullptr;
  int64_t col_cap = 0;
  int DM = 0;                    // largest active frame distance of the radius table
  int32_t* runs = nullptr;       // per query tile: key-tile column runs per (frame, tile row)
  int32_t* rowwin = nullptr;     // per query tile: first frame | frames << 16
  int32_t* glist = nullptr;  // bf16 only: merged tile lists of query-tile groups, 2 int32 per entry
  int64_t glist_cap = 0;     // entries
  int32_t* glen = nullptr;   // per group: list length
  int32_t* gptr = nullptr;   // per group: list offset (exclusive scan of glen)
  int64_t n_groups = 0;
  int group_rows = 0;        // bf16: query-tile rows per group (2 or 3)
  uint8_t* perm = nullptr;   // regroup: per group, its query slots in level order (GROUP_SLOTS each)
  int64_t* totals = nullptr;      // device: nnz, longest row, overflow flag (+4: groups, +8: filtered CSR)
  // vote threshold > 1: per-entry votes of the unfiltered CSR, the filtered CSR's
  // second buffers (swapped in after filtering) and the retained-pair count
  int16_t* votes = nullptr;
  int64_t votes_cap = 0;
  int32_t* row_ptr2 = nullptr;
  int32_t* col_idx2 = nullptr;
  int64_t col2_cap = 0;
  unsigned long long* kept_votes = nullptr;  // device
  int64_t retained_votes = 0;
  int64_t* totals_host = nullptr; // pinned, 8 entries
  int64_t nnz = 0;
  int32_t max_row_len = 0;
  // Scratch owned by the plan for tra_plan_stats and tra_plan_drift, so that
  // neither allocates per call: two pair counters and a level-difference
  // counter, and (entropy plans) the pooled keys and levels of the inputs a
  // drift query measures.
  unsigned long long* counters = nullptr;  // device, 4 entries
  void* kbar2 = nullptr;
  int16_t* lv2 = nullptr;
  // Set by a build that completed; cleared when a build starts, so a plan
  // whose last build failed is refused by the calls that read it.
  bool valid = false;
  // bf16 plans without a vote threshold build only what the attention kernel
  // reads (levels, the per-row runs and counts, the group lists, into a
  // group-list buffer sized for the worst case at creation), so a build
  // neither allocates nor waits for the device.  Their CSR is completed from
  // the counts and runs on first use (export, stats, info).
  bool lazy_csr = false;
  bool csr_ready = false;
  int64_t glist_stride = 0;  // lazy-CSR plans: group g's list starts at entry g * glist_stride
  hipEvent_t built = nullptr;  // recorded at the end of each build
};

namespace {

void release(tra_plan* p) {
  if (!p) return;
  void* bufs[] = {p->kbar, p->H, p->lv, p->r2, p->dmax, p->r2c, p->r2off, p->pool_w,
                  p->counts, p->row_ptr, p->col_idx, p->runs, p->rowwin, p->glist, p->glen, p->gptr, p->totals, p->votes,
                  p->row_ptr2, p->col_idx2, p->kept_votes, p->counters, p->kbar2, p->lv2, p->perm};
  for (void* b : bufs)
    if (b) (void)hipFree(b);
  if (p->totals_host) (void)hipHostFree(p->totals_host);
  if (p->built) (void)hipEventDestroy(p->built);
  delete p;
}

tra::RadiusTable radius_table_of(const tra_plan* p) {
  return tra::RadiusTable{p->r2, p->dmax, p->r2c, p->r2off, static_cast<int>(p->table.r2c.size()), p->shape.T,
                          metric_of(p->params)};
}

// Query-tile rows per group of the bf16 attention kernel.  A group of 3 x 2
// query tiles shares each key tile among 384 queries and puts three waves on
// every SIMD, which overlap one another's matrix and vector phases better
// than two.  It is taken unless it would leave more tile rows of the grid
// empty than 2 x 2 groups, the plan regroups queries (a 2 x 2 layout), or the
// 1-D window generator is used (its masks need more registers than three
// waves per SIMD leave at head_dim 128).
int group_rows_for(const tra_params& p, const tra::Grid& tiles) {
  if (p.group_rows) return p.group_rows;
  if (p.regroup || p.generator == TRA_GEN_WINDOW_1D) return 2;
  const int pad3 = (3 - tiles.nh % 3) % 3, pad2 = tiles.nh % 2;
  return pad3 <= pad2 ? 3 : 2;
}

tra_status build_lists(tra_plan* p, hipStream_t st);

// Steps entropy -> level -> tile lists into the plan's buffers.  The levels
// come from the pooled-key entropy of (q, k), or, when `Hin` is not NULL, from
// the given per-query entropies.
tra_status build(tra_plan* p, const void* q, const void* k, const float* Hin, hipStream_t st) {
  p->valid = false;
  const tra_shape& s = p->shape;
  const int d = s.head_dim;
  Range r_all("tra.plan");
  {
    Range r("tra.plan.levels");
    if (p->params.radius_override < 0.0) {
      tra::EntropyArgs ea{p->params.a, p->params.c, p->params.levels_per_nat, p->table.k_lo, p->table.k_hi};
      if (Hin) {
        TRA_LAUNCH(tra::launch_levels_from_entropy(Hin, p->n_queries, ea, p->H, p->lv, st));
      } else {
        TRA_LAUNCH(tra::launch_pool(s.dtype, d, k, p->kbar, p->BH, p->pool, st));
        TRA_LAUNCH(tra::launch_entropy(s.dtype, d, q, p->kbar, p->pool_w, p->BH, static_cast<int>(p->N),
                                       p->pool, ea, p->H, p->lv, st));
      }
    } else {
      TRA_LAUNCH(tra::launch_fill_levels(p->lv, p->H, p->n_queries, st));
    }
  }
  const tra_status ls = build_lists(p, st);
  if (ls != TRA_OK) return ls;
  p->valid = true;
  return TRA_OK;
}

// Group lists only (lazy-CSR plans): runs and per-row counts, then the
// merged lists of the groups, with no host round trip.
tra_status build_group_lists_only(tra_plan* p, hipStream_t st) {
  const tra_shape& s = p->shape;
  p->csr_ready = false;
  // Each group writes its list into its own fixed slot (gptr[g] = g * stride,
  // set at creation) and its length to glen: no counting pass, no scan.
  if (p->params.generator == TRA_GEN_WINDOW_1D) {
    TRA_LAUNCH(tra::launch_window_groups(true, p->lv, p->r2, p->dmax, s.T, p->row_base, p->BH, p->tiles,
                                      p->group_rows, p->gptr, p->glist, p->glen, st));
  } else {
    // One pass: each workgroup writes the runs of a group's tiles, then the group's list.
    TRA_LAUNCH(tra::launch_csr_runs(p->params.generator == TRA_GEN_MANHATTAN, p->lv, radius_table_of(p),
                                    p->table.n_levels, p->row_base, p->BH, p->tiles, p->DM, p->counts, p->runs,
                                    p->rowwin, st, p->group_rows, p->gptr, p->glist, p->glen));
  }
  TRA_HIP(hipEventRecord(p->built, st));
  return TRA_OK;
}

// Completes the CSR of a lazy-CSR plan (on `st`, after its last build), once
// per build.  Synchronises `st`.
tra_status ensure_csr(tra_plan* p, hipStream_t st) {
  if (!p->lazy_csr || p->csr_ready) return TRA_OK;
  Range r("tra.plan.csr");
  const tra_shape& s = p->shape;
  const bool window = p->params.generator == TRA_GEN_WINDOW_1D;
  TRA_HIP(hipStreamWaitEvent(st, p->built, 0));
  if (window)
    TRA_LAUNCH(tra::launch_window_csr(false, p->lv, p->r2, p->dmax, s.T, p->row_base, p->BH, p->tiles, nullptr,
                                   p->counts, nullptr, st));
  TRA_LAUNCH(tra::launch_scan(p->counts, p->n_rows, p->row_ptr, p->totals, st));
  TRA_HIP(hipMemcpyAsync(p->totals_host, p->totals, 3 * sizeof(int64_t), hipMemcpyDeviceToHost, st));
  TRA_HIP(hipStreamSynchronize(st));
  if (p->totals_host[2]) return fail(TRA_ERR_OVERFLOW, "CSR has 2^31 or more entries");
  p->nnz = p->totals_host[0];
  p->max_row_len = static_cast<int32_t>(p->totals_host[1]);
  if (p->nnz > p->col_cap) {
    if (p->col_idx) TRA_HIP(hipFree(p->col_idx));
    p->col_idx = nullptr;
    p->col_cap = 0;
    const int64_t cap = p->nnz + p->nnz / 8 + 64;
    TRA_HIP(dev_alloc(&p->col_idx, cap * sizeof(int32_t)));
    p->col_cap = cap;
  }
  if (window)
    TRA_LAUNCH(tra::launch_window_csr(true, p->lv, p->r2, p->dmax, s.T, p->row_base, p->BH, p->tiles, p->row_ptr,
                                   p->counts, p->col_idx, st));
  else
    TRA_LAUNCH(tra::launch_csr_expand(p->BH, p->tiles, p->DM, p->runs, p->rowwin, p->row_ptr, p->col_idx, st));
  TRA_HIP(hipStreamSynchronize(st));
  p->csr_ready = true;
  return TRA_OK;
}

// Tile lists (CSR, votes, group lists) from the levels in p->lv.
tra_status build_lists(tra_plan* p, hipStream_t st) {
  Range r_lists("tra.plan.tile_lists");
  if (p->perm) TRA_LAUNCH(tra::launch_regroup(p->lv, p->BH, p->tiles, p->perm, st));
  if (p->lazy_csr) return build_group_lists_only(p, st);
  const tra_shape& s = p->shape;
  const bool window = p->params.generator == TRA_GEN_WINDOW_1D;
  if (window) {
    TRA_LAUNCH(tra::launch_window_csr(false, p->lv, p->r2, p->dmax, s.T, p->row_base, p->BH, p->tiles, nullptr,
                                   p->counts, nullptr, st));
  } else {
    TRA_LAUNCH(tra::launch_csr_runs(p->params.generator == TRA_GEN_MANHATTAN, p->lv, radius_table_of(p),
                                    p->table.n_levels, p->row_base, p->BH, p->tiles, p->DM, p->counts, p->runs,
                                    p->rowwin, st));
  }
  TRA_LAUNCH(tra::launch_scan(p->counts, p->n_rows, p->row_ptr, p->totals, st));
  TRA_HIP(hipMemcpyAsync(p->totals_host, p->totals, 3 * sizeof(int64_t), hipMemcpyDeviceToHost, st));
  TRA_HIP(hipStreamSynchronize(st));
  if (p->totals_host[2]) return fail(TRA_ERR_OVERFLOW, "CSR has 2^31 or more entries");
  p->nnz = p->totals_host[0];
  p->max_row_len = static_cast<int32_t>(p->totals_host[1]);
  if (p->nnz > p->col_cap) {
    if (p->col_idx) TRA_HIP(hipFree(p->col_idx));
    p->col_idx = nullptr;
    p->col_cap = 0;
    const int64_t cap = p->nnz + p->nnz / 8 + 64;
    TRA_HIP(dev_alloc(&p->col_idx, cap * sizeof(int32_t)));
    p->col_cap = cap;
  }
  if (window) {
    TRA_LAUNCH(tra::launch_window_csr(true, p->lv, p->r2, p->dmax, s.T, p->row_base, p->BH, p->tiles, p->row_ptr,
                                   p->counts, p->col_idx, st));
  } else {
    TRA_LAUNCH(tra::launch_csr_expand(p->BH, p->tiles, p->DM, p->runs, p->rowwin, p->row_ptr, p->col_idx, st));
  }
  const int theta = p->params.vote_threshold;
  const bool l1 = p->params.generator == TRA_GEN_MANHATTAN;
  if (theta > 1) {
    // Token voting with a threshold: votes per entry, then the entries with at
    // least theta votes form the plan's CSR.
    Range r("tra.plan.votes");
    if (p->nnz > p->votes_cap) {
      if (p->votes) TRA_HIP(hipFree(p->votes));
      p->votes = nullptr;
      p->votes_cap = 0;
      TRA_HIP(dev_alloc(&p->votes, p->col_cap * sizeof(int16_t)));
      p->votes_cap = p->col_cap;
    }
    TRA_HIP(hipMemsetAsync(p->kept_votes, 0, sizeof(unsigned long long), st));
    TRA_LAUNCH(tra::launch_votes(l1, p->lv, p->r2, p->dmax, s.T, p->row_base, p->BH, p->tiles, p->row_ptr, p->col_idx,
                              theta, p->votes, p->counts, p->kept_votes, st));
    TRA_LAUNCH(tra::launch_scan(p->counts, p->n_rows, p->row_ptr2, p->totals + 8, st));
    TRA_HIP(hipMemcpyAsync(p->totals_host, p->totals + 8, 2 * sizeof(int64_t), hipMemcpyDeviceToHost, st));
    TRA_HIP(hipMemcpyAsync(p->totals_host + 2, p->kept_votes, sizeof(int64_t), hipMemcpyDeviceToHost, st));
    TRA_HIP(hipStreamSynchronize(st));
    const int64_t nnz2 = p->totals_host[0];
    if (nnz2 > p->col2_cap) {
      if (p->col_idx2) TRA_HIP(hipFree(p->col_idx2));
      p->col_idx2 = nullptr;
      p->col2_cap = 0;
      const int64_t cap = nnz2 + nnz2 / 8 + 64;
      TRA_HIP(dev_alloc(&p->col_idx2, cap * sizeof(int32_t)));
      p->col2_cap = cap;
    }
    TRA_LAUNCH(tra::launch_vote_compact(p->n_rows, p->row_ptr, p->col_idx, p->votes, theta, p->row_ptr2, p->col_idx2,
                                     st));
    std::swap(p->row_ptr, p->row_ptr2);
    std::swap(p->col_idx, p->col_idx2);
    std::swap(p->col_cap, p->col2_cap);
    p->nnz = nnz2;
    p->max_row_len = static_cast<int32_t>(p->totals_host[1]);
    p->retained_votes = p->totals_host[2];
  }
  if (s.dtype == TRA_BF16) {
    Range r("tra.plan.group_lists");
    if (p->nnz > p->glist_cap) {
      if (p->glist) TRA_HIP(hipFree(p->glist));
      p->glist = nullptr;
      p->glist_cap = 0;
      TRA_HIP(dev_alloc(&p->glist, p->col_cap * 2 * sizeof(int32_t)));
      p->glist_cap = p->col_cap;
    }
    if (window) {
      TRA_LAUNCH(tra::launch_window_groups(false, p->lv, p->r2, p->dmax, s.T, p->row_base, p->BH, p->tiles,
                                        p->group_rows, nullptr, nullptr, p->glen, st));
      TRA_LAUNCH(tra::launch_scan(p->glen, p->n_groups, p->gptr, p->totals + 4, st));
      TRA_LAUNCH(tra::launch_window_groups(true, p->lv, p->r2, p->dmax, s.T, p->row_base, p->BH, p->tiles,
                                        p->group_rows, p->gptr, p->glist, p->glen, st));
    } else {
      const int32_t* frp = theta > 1 ? p->row_ptr : nullptr;
      TRA_LAUNCH(tra::launch_group_lists(false, p->BH, p->tiles, p->group_rows, p->DM, p->runs, p->rowwin, frp,
                                      p->col_idx, nullptr, nullptr, p->glen, st));
      TRA_LAUNCH(tra::launch_scan(p->glen, p->n_groups, p->gptr, p->totals + 4, st));
      TRA_LAUNCH(tra::launch_group_lists(true, p->BH, p->tiles, p->group_rows, p->DM, p->runs, p->rowwin, frp,
                                      p->col_idx, p->gptr, p->glist, p->glen, st));
    }
  }
  TRA_HIP(hipEventRecord(p->built, st));  // the host-copy calls wait for it
  return TRA_OK;
}

}  // namespace

extern "C" {

tra_status tra_params_validate(const tra_shape* shape, const tra_params* params) {
  tra_status st = check_shape(shape);
  if (st != TRA_OK) return st;
  return check_params(shape, params, nullptr);
}

tra_status tra_radius_table(const tra_shape* shape, const tra_params* params, int32_t* r2,
                            double* r0sq, int32_t* n_levels, int32_t* k_lo) {
  tra_status st = check_shape(shape);
  if (st != TRA_OK) return st;
  Table t;
  st = check_params(shape, params, &t);
  if (st != TRA_OK) return st;
  if (n_levels) *n_levels = t.n_levels;
  if (k_lo) *k_lo = t.k_lo;
  if (r2) std::memcpy(r2, t.r2.data(), t.r2.size() * sizeof(int32_t));
  if (r0sq) std::memcpy(r0sq, t.r0sq.data(), t.r0sq.size() * sizeof(double));
  return TRA_OK;
}

}  // extern "C"

namespace {

// Validated shape and params -> a plan with every buffer allocated and the
// radius table uploaded, levels and tile lists not yet built.
tra_status create_plan(const tra_shape* shape, const tra_params* params, Table&& tab, hipStream_t hs,
                       tra_plan** out) {
  tra_plan* p = new tra_plan();
  p->shape = *shape;
  p->params = *params;
  p->table = std::move(tab);
  p->BH = shape->B * shape->heads;
  p->N = static_cast<int64_t>(shape->T) * shape->H * shape->W;
  p->n_queries = p->BH * p->N;
  p->pool = tra::make_grid(shape->T, shape->H, shape->W, params->pool_h, params->pool_w);
  p->tiles = tra::make_grid(shape->T, shape->H, shape->W, params->tile_h, params->tile_w);
  p->n_rows = static_cast<int64_t>(p->BH) * p->tiles.count;
  p->row_base = params->radius_override >= 0.0 ? -1 : p->table.k_lo;

  auto fin = [&](tra_status s2) {
    if (s2 != TRA_OK) release(p);
    return s2;
  };
#define TRA_HIP_P(call)                                                                       \
  do {                                                                                        \
    hipError_t e_ = (call);                                                                   \
    if (e_ != hipSuccess)                                                                     \
      return fin(fail(e_ == hipErrorOutOfMemory ? TRA_ERR_OOM : TRA_ERR_HIP,                  \
                      std::string(#call) + ": " + hipGetErrorString(e_)));                     \
  } while (0)

  const size_t es = dtype_size(shape->dtype);
  TRA_HIP_P(dev_alloc(&p->kbar, static_cast<size_t>(p->BH) * p->pool.count * shape->head_dim * es));
  TRA_HIP_P(dev_alloc(&p->H, p->n_queries * sizeof(float)));
  TRA_HIP_P(dev_alloc(&p->lv, p->n_queries * sizeof(int16_t)));
  TRA_HIP_P(dev_alloc(&p->r2, p->table.r2.size() * sizeof(int32_t)));
  TRA_HIP_P(dev_alloc(&p->dmax, p->table.dmax.size() * sizeof(int32_t)));
  TRA_HIP_P(dev_alloc(&p->r2c, p->table.r2c.size() * sizeof(int32_t)));
  TRA_HIP_P(dev_alloc(&p->r2off, p->table.r2off.size() * sizeof(int32_t)));
  TRA_HIP_P(dev_alloc(&p->pool_w, static_cast<size_t>(p->pool.count) * sizeof(float)));
  TRA_HIP_P(dev_alloc(&p->counts, p->n_rows * sizeof(int32_t)));
  TRA_HIP_P(dev_alloc(&p->row_ptr, (p->n_rows + 1) * sizeof(int32_t)));
  TRA_HIP_P(dev_alloc(&p->totals, 12 * sizeof(int64_t)));
  if (params->vote_threshold > 1) {
    TRA_HIP_P(dev_alloc(&p->row_ptr2, (p->n_rows + 1) * sizeof(int32_t)));
    TRA_HIP_P(dev_alloc(&p->kept_votes, sizeof(unsigned long long)));
  }
  for (int32_t dm : p->table.dmax) p->DM = std::max(p->DM, static_cast<int>(dm));
  if (params->generator != TRA_GEN_WINDOW_1D) {  // the window builds its lists without runs
    const int64_t run_entries = p->n_rows * (2 * p->DM + 1) * p->tiles.nh;
    if (run_entries > (int64_t(1) << 32)) return fin(fail(TRA_ERR_SHAPE, "tile-list run buffer too large"));
    TRA_HIP_P(dev_alloc(&p->runs, run_entries * sizeof(int32_t)));
    TRA_HIP_P(dev_alloc(&p->rowwin, p->n_rows * sizeof(int32_t)));
  }
  if (shape->dtype == TRA_BF16) {
    p->group_rows = group_rows_for(*params, p->tiles);
    p->n_groups = tra::group_count(p->BH, p->tiles, p->group_rows);
    TRA_HIP_P(dev_alloc(&p->glen, p->n_groups * sizeof(int32_t)));
    if (params->regroup) TRA_HIP_P(dev_alloc(&p->perm, p->n_groups * tra::GROUP_SLOTS));
    TRA_HIP_P(dev_alloc(&p->gptr, (p->n_groups + 1) * sizeof(int32_t)));
    // A group's list holds at most every key tile of the frames within the
    // table's reach of its own frame.
    const int64_t per_group =
        static_cast<int64_t>(std::min(shape->T, 2 * p->DM + 1)) * p->tiles.per_frame;
    const int64_t bound = p->n_groups * per_group;
    if (params->vote_threshold <= 1 && bound * 8 <= (int64_t(1) << 32)) {
      p->lazy_csr = true;
      TRA_HIP_P(dev_alloc(&p->glist, bound * 2 * sizeof(int32_t)));
      p->glist_cap = bound;
      p->glist_stride = per_group;
      std::vector<int32_t> slots(p->n_groups + 1);
      for (int64_t g = 0; g <= p->n_groups; ++g) slots[g] = static_cast<int32_t>(g * per_group);
      TRA_HIP_P(hipMemcpy(p->gptr, slots.data(), slots.size() * sizeof(int32_t), hipMemcpyHostToDevice));
    }
  }
  // Recorded at the end of every build; the calls that copy plan data to the
  // host wait for it on their own stream.
  TRA_HIP_P(hipEventCreateWithFlags(&p->built, hipEventDisableTiming));
  TRA_HIP_P(host_alloc(&p->totals_host, 8 * sizeof(int64_t)));
  TRA_HIP_P(dev_alloc(&p->counters, 4 * sizeof(unsigned long long)));
  if (params->radius_override < 0.0) {
    TRA_HIP_P(dev_alloc(&p->kbar2, static_cast<size_t>(p->BH) * p->pool.count * shape->head_dim * es));
    TRA_HIP_P(dev_alloc(&p->lv2, p->n_queries * sizeof(int16_t)));
  }
  TRA_HIP_P(hipGetDevice(&p->device));

  std::vector<float> w(p->pool.count);  // in the pooled keys' storage order
  for (int b = 0; b < p->pool.count; ++b) {
    const int rem = b % p->pool.per_frame;
    const int h0 = (rem / p->pool.nw) * p->pool.th, w0 = (rem % p->pool.nw) * p->pool.tw;
    w[tra::pool_pos(p->pool, b)] =
        static_cast<float>(std::min(p->pool.th, shape->H - h0) * std::min(p->pool.tw, shape->W - w0));
  }
  TRA_HIP_P(hipMemcpy(p->r2, p->table.r2.data(), p->table.r2.size() * sizeof(int32_t), hipMemcpyHostToDevice));
  TRA_HIP_P(hipMemcpy(p->dmax, p->table.dmax.data(), p->table.dmax.size() * sizeof(int32_t), hipMemcpyHostToDevice));
  TRA_HIP_P(hipMemcpy(p->pool_w, w.data(), w.size() * sizeof(float), hipMemcpyHostToDevice));
  TRA_HIP_P(hipMemcpy(p->r2c, p->table.r2c.data(), p->table.r2c.size() * sizeof(int32_t), hipMemcpyHostToDevice));
  TRA_HIP_P(hipMemcpy(p->r2off, p->table.r2off.data(), p->table.r2off.size() * sizeof(int32_t), hipMemcpyHostToDevice));
  // Pooled keys stay zero until a build from (q, k) writes them.
  TRA_HIP_P(hipMemsetAsync(p->kbar, 0, static_cast<size_t>(p->BH) * p->pool.count * shape->head_dim * es, hs));
#undef TRA_HIP_P
  *out = p;
  return TRA_OK;
}

tra_status check_qk(const void* q, const void* k) {
  if (!q || !k) return fail(TRA_ERR_INVALID_ARG, "q and k must be device pointers");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k)) & 15)
    return fail(TRA_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
  return TRA_OK;
}

tra_status check_entropy_ptr(const float* H) {
  if (!H) return fail(TRA_ERR_INVALID_ARG, "entropy must be a device pointer");
  if (reinterpret_cast<uintptr_t>(H) & 3) return fail(TRA_ERR_INVALID_ARG, "entropy must be 4-byte aligned");
  return TRA_OK;
}

}  // namespace

namespace tra {

size_t drift_scratch_bytes(const tra_plan* p) {
  if (p->params.radius_override >= 0.0) return 0;
  const size_t kbar = static_cast<size_t>(p->BH) * p->pool.count * p->shape.head_dim * dtype_size(p->shape.dtype);
  const size_t lv = static_cast<size_t>(p->n_queries) * sizeof(int16_t);
  return scratch_round(kbar) + scratch_round(lv) + scratch_round(sizeof(unsigned long long));
}

void drift_scratch_layout(const tra_plan* p, unsigned char* base, void** kbar, int16_t** lv,
                          unsigned long long** counter) {
  const size_t kb = static_cast<size_t>(p->BH) * p->pool.count * p->shape.head_dim * dtype_size(p->shape.dtype);
  const size_t lb = static_cast<size_t>(p->n_queries) * sizeof(int16_t);
  *kbar = base;
  *lv = reinterpret_cast<int16_t*>(base + scratch_round(kb));
  *counter = reinterpret_cast<unsigned long long*>(base + scratch_round(kb) + scratch_round(lb));
}

int plan_device(const tra_plan* p) { return p->device; }

tra_status report(tra_status s, const std::string& msg) { return fail(s, msg); }

tra_status drift_with_scratch(const tra_plan* plan, const void* q, const void* k, void* kbar, int16_t* lv,
                              unsigned long long* counter, int64_t* changed, void* stream) {
  if (!plan || !changed) return fail(TRA_ERR_INVALID_ARG, "plan and changed must not be NULL");
  if (!plan->valid) return fail(TRA_ERR_PLAN_INVALID, "the plan's last build failed");
  tra_status st = check_qk(q, k);
  if (st != TRA_OK) return st;
  *changed = 0;
  if (plan->params.radius_override >= 0.0) return TRA_OK;
  fault_arm();
  const tra_shape& s = plan->shape;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  int64_t* host = plan->totals_host + 6;  // the plan's pinned word for the count
  const EntropyArgs ea{plan->params.a, plan->params.c, plan->params.levels_per_nat, plan->table.k_lo,
                       plan->table.k_hi};
  TRA_LAUNCH(launch_clear_counters(counter, 1, hs));
  TRA_LAUNCH(launch_pool(s.dtype, s.head_dim, k, kbar, plan->BH, plan->pool, hs));
  TRA_LAUNCH(launch_entropy(s.dtype, s.head_dim, q, kbar, plan->pool_w, plan->BH, static_cast<int>(plan->N),
                            plan->pool, ea, nullptr, lv, hs));
  TRA_LAUNCH(launch_level_diff(plan->lv, lv, plan->n_queries, counter, hs));
  TRA_HIP(hipMemcpyAsync(host, counter, sizeof(unsigned long long), hipMemcpyDeviceToHost, hs));
  TRA_HIP(hipStreamSynchronize(hs));
  *changed = *host;
  return TRA_OK;
}

}  // namespace tra

extern "C" {

tra_status tra_plan_create(const tra_shape* shape, const tra_params* params, const void* q,
                           const void* k, void* stream, tra_plan** out) {
  if (!out) return fail(TRA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  fault_arm();
  tra_status st = check_shape(shape);
  if (st != TRA_OK) return st;
  Table tab;
  st = check_params(shape, params, &tab);
  if (st != TRA_OK) return st;
  st = check_qk(q, k);
  if (st != TRA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  tra_plan* p = nullptr;
  st = create_plan(shape, params, std::move(tab), hs, &p);
  if (st != TRA_OK) return st;
  st = build(p, q, k, nullptr, hs);
  if (st != TRA_OK) {
    release(p);
    return st;
  }
  *out = p;
  return TRA_OK;
}

tra_status tra_plan_create_from_entropy(const tra_shape* shape, const tra_params* params,
                                        const float* entropy, void* stream, tra_plan** out) {
  if (!out) return fail(TRA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  fault_arm();
  tra_status st = check_shape(shape);
  if (st != TRA_OK) return st;
  Table tab;
  st = check_params(shape, params, &tab);
  if (st != TRA_OK) return st;
  st = check_entropy_ptr(entropy);
  if (st != TRA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  tra_plan* p = nullptr;
  st = create_plan(shape, params, std::move(tab), hs, &p);
  if (st != TRA_OK) return st;
  st = build(p, nullptr, nullptr, entropy, hs);
  if (st != TRA_OK) {
    release(p);
    return st;
  }
  *out = p;
  return TRA_OK;
}

tra_status tra_plan_rebuild_from_entropy(tra_plan* plan, const float* entropy, void* stream) {
  if (!plan) return fail(TRA_ERR_INVALID_ARG, "plan is NULL");
  const tra_status st = check_entropy_ptr(entropy);
  if (st != TRA_OK) return st;
  fault_arm();
  return build(plan, nullptr, nullptr, entropy, static_cast<hipStream_t>(stream));
}

tra_status tra_plan_import(const tra_shape* shape, const tra_params* params, const int16_t* levels,
                           const float* entropy, const void* kbar, void* stream, tra_plan** out) {
  if (!out) return fail(TRA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  fault_arm();
  tra_status st = check_shape(shape);
  if (st != TRA_OK) return st;
  Table tab;
  st = check_params(shape, params, &tab);
  if (st != TRA_OK) return st;
  if (!levels) return fail(TRA_ERR_INVALID_ARG, "levels is NULL");
  // Every level must name a row of the radius table (-1 under radius_override).
  const int64_t nq = static_cast<int64_t>(shape->B) * shape->heads * shape->T * shape->H * shape->W;
  const bool fixed = params->radius_override >= 0.0;
  const int lo = fixed ? -1 : tab.k_lo, hi = fixed ? -1 : tab.k_lo + tab.n_levels - 1;
  for (int64_t i = 0; i < nq; ++i)
    if (levels[i] < lo || levels[i] > hi)
      return fail(TRA_ERR_INVALID_ARG, "level " + std::to_string(levels[i]) + " of query " + std::to_string(i) +
                                           " outside [" + std::to_string(lo) + ", " + std::to_string(hi) + "]");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  Range r("tra.plan.import");
  tra_plan* p = nullptr;
  st = create_plan(shape, params, std::move(tab), hs, &p);
  if (st != TRA_OK) return st;
  auto fin = [&](tra_status s2) {
    if (s2 != TRA_OK) release(p);
    return s2;
  };
#define TRA_HIP_I(call)                                                                       \
  do {                                                                                        \
    hipError_t e_ = (call);                                                                   \
    if (e_ != hipSuccess)                                                                     \
      return fin(fail(TRA_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_)));       \
  } while (0)
  // create_plan queued the clearing of the pooled keys on hs; copies go after it.
  TRA_HIP_I(hipStreamSynchronize(hs));
  TRA_HIP_I(hipMemcpy(p->lv, levels, nq * sizeof(int16_t), hipMemcpyHostToDevice));
  if (entropy) TRA_HIP_I(hipMemcpy(p->H, entropy, nq * sizeof(float), hipMemcpyHostToDevice));
  else TRA_HIP_I(hipMemsetAsync(p->H, 0, nq * sizeof(float), hs));
  if (kbar) {
    // ABI order (raster over the pool rectangles) -> storage order
    const size_t row = static_cast<size_t>(shape->head_dim) * dtype_size(shape->dtype);
    std::vector<char> tmp(static_cast<size_t>(p->BH) * p->pool.count * row);
    for (int bh = 0; bh < p->BH; ++bh)
      for (int b = 0; b < p->pool.count; ++b)
        std::memcpy(&tmp[(static_cast<size_t>(bh) * p->pool.count + tra::pool_pos(p->pool, b)) * row],
                    static_cast<const char*>(kbar) + (static_cast<size_t>(bh) * p->pool.count + b) * row, row);
    TRA_HIP_I(hipMemcpy(p->kbar, tmp.data(), tmp.size(), hipMemcpyHostToDevice));
  }
#undef TRA_HIP_I
  st = build_lists(p, hs);
  if (st != TRA_OK) return fin(st);
  p->valid = true;
  *out = p;
  return TRA_OK;
}

tra_status tra_dense_attention(const tra_shape* shape, const void* q, const void* k, const void* v,
                               void* o, float* entropy, void* stream) {
  tra_status st = check_shape(shape);
  if (st != TRA_OK) return st;
  if (shape->dtype == TRA_BF16 &&
      static_cast<int64_t>(shape->T) * shape->H * shape->W * shape->head_dim * 2 >= (int64_t(1) << 31))
    return fail(TRA_ERR_SHAPE, "bf16 attention needs T*H*W*head_dim*2 (bytes of one head) below 2^31");
  if (!q || !k || !v || !o) return fail(TRA_ERR_INVALID_ARG, "q, k, v and o must be device pointers");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
       reinterpret_cast<uintptr_t>(o)) & 15)
    return fail(TRA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (o == q || o == k || o == v) return fail(TRA_ERR_INVALID_ARG, "o must not alias q, k or v");
  if (entropy && (reinterpret_cast<uintptr_t>(entropy) & 3))
    return fail(TRA_ERR_INVALID_ARG, "entropy must be 4-byte aligned");
  const int BH = shape->B * shape->heads;
  const int N = shape->T * shape->H * shape->W;
  fault_arm();
  Range r("tra.dense_attention");
  TRA_LAUNCH(tra::launch_dense(shape->dtype, shape->head_dim, q, k, v, o, entropy, BH, N,
                            static_cast<hipStream_t>(stream)));
  return TRA_OK;
}

tra_status tra_attention(const tra_plan* plan, const void* q, const void* k, const void* v,
                         void* o, void* stream) {
  if (!plan) return fail(TRA_ERR_INVALID_ARG, "plan is NULL");
  if (!q || !k || !v || !o) return fail(TRA_ERR_INVALID_ARG, "q, k, v and o must be device pointers");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
       reinterpret_cast<uintptr_t>(o)) & 15)
    return fail(TRA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (o == q || o == k || o == v) return fail(TRA_ERR_INVALID_ARG, "o must not alias q, k or v");
  if (!plan->valid) return fail(TRA_ERR_PLAN_INVALID, "the plan's last build failed");
  fault_arm();
  Range r("tra.attention");
  const tra_shape& s = plan->shape;
  const tra::RadiusTable tab = radius_table_of(plan);
  TRA_LAUNCH(tra::launch_attention(s.dtype, s.head_dim, q, k, v, o, plan->lv, tab, plan->row_base,
                                plan->BH, plan->tiles, plan->row_ptr, plan->col_idx,
                                plan->gptr, plan->glist, plan->glen, plan->group_rows, plan->perm,
                                plan->params.block_mask != 0,
                                plan->params.vote_threshold == 1, static_cast<hipStream_t>(stream)));
  return TRA_OK;
}

tra_status tra_plan_rebuild(tra_plan* plan, const void* q, const void* k, void* stream) {
  if (!plan) return fail(TRA_ERR_INVALID_ARG, "plan is NULL");
  const tra_status st = check_qk(q, k);
  if (st != TRA_OK) return st;
  fault_arm();
  return build(plan, q, k, nullptr, static_cast<hipStream_t>(stream));
}

tra_status tra_plan_matches(const tra_plan* plan, const tra_shape* shape) {
  if (!plan || !shape) return fail(TRA_ERR_INVALID_ARG, "plan and shape must not be NULL");
  const tra_shape& s = plan->shape;
  if (s.B != shape->B || s.heads != shape->heads || s.T != shape->T || s.H != shape->H ||
      s.W != shape->W || s.head_dim != shape->head_dim || s.dtype != shape->dtype)
    return fail(TRA_ERR_PLAN_MISMATCH, "tensor shape or dtype differs from the plan's");
  return TRA_OK;
}

tra_status tra_plan_get_info(const tra_plan* plan, tra_plan_info* info) {
  if (!plan || !info) return fail(TRA_ERR_INVALID_ARG, "plan and info must not be NULL");
  if (plan->valid) {  // nnz and the longest row come with the CSR (null stream)
    fault_arm();
    const tra_status st = ensure_csr(const_cast<tra_plan*>(plan), nullptr);
    if (st != TRA_OK) return st;
  }
  info->n_queries = plan->n_queries;
  info->n_rows = plan->n_rows;
  info->nnz = plan->nnz;
  info->n_qtiles = plan->tiles.count;
  info->n_pool = plan->pool.count;
  info->n_levels = plan->table.n_levels;
  info->k_lo = plan->table.k_lo;
  info->T = plan->shape.T;
  info->max_row_len = plan->max_row_len;
  info->group_rows = plan->group_rows;
  return TRA_OK;
}

tra_status tra_plan_export(const tra_plan* plan, int16_t* levels, float* entropy, int32_t* r2,
                           int32_t* row_ptr, int32_t* col_idx, void* kbar, void* stream) {
  if (!plan) return fail(TRA_ERR_INVALID_ARG, "plan is NULL");
  if (!plan->valid) return fail(TRA_ERR_PLAN_INVALID, "the plan's last build failed");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (row_ptr || col_idx) {
    fault_arm();
    const tra_status st = ensure_csr(const_cast<tra_plan*>(plan), hs);
    if (st != TRA_OK) return st;
  }
  // An asynchronous build may still run on another stream.
  if (plan->built) TRA_HIP(hipStreamWaitEvent(hs, plan->built, 0));
  TRA_HIP(hipStreamSynchronize(hs));
  if (levels) TRA_HIP(hipMemcpy(levels, plan->lv, plan->n_queries * sizeof(int16_t), hipMemcpyDeviceToHost));
  if (entropy) TRA_HIP(hipMemcpy(entropy, plan->H, plan->n_queries * sizeof(float), hipMemcpyDeviceToHost));
  if (r2) std::memcpy(r2, plan->table.r2.data(), plan->table.r2.size() * sizeof(int32_t));
  if (row_ptr) TRA_HIP(hipMemcpy(row_ptr, plan->row_ptr, (plan->n_rows + 1) * sizeof(int32_t), hipMemcpyDeviceToHost));
  if (col_idx && plan->nnz > 0)
    TRA_HIP(hipMemcpy(col_idx, plan->col_idx, plan->nnz * sizeof(int32_t), hipMemcpyDeviceToHost));
  if (kbar) {
    // storage order (full rectangles first) -> ABI order (raster)
    const size_t row = static_cast<size_t>(plan->shape.head_dim) * dtype_size(plan->shape.dtype);
    std::vector<char> tmp(static_cast<size_t>(plan->BH) * plan->pool.count * row);
    TRA_HIP(hipMemcpy(tmp.data(), plan->kbar, tmp.size(), hipMemcpyDeviceToHost));
    for (int bh = 0; bh < plan->BH; ++bh)
      for (int b = 0; b < plan->pool.count; ++b)
        std::memcpy(static_cast<char*>(kbar) + (static_cast<size_t>(bh) * plan->pool.count + b) * row,
                    &tmp[(static_cast<size_t>(bh) * plan->pool.count + tra::pool_pos(plan->pool, b)) * row], row);
  }
  return TRA_OK;
}

tra_status tra_plan_export_regroup(const tra_plan* plan, uint8_t* perm, void* stream) {
  if (!plan || !perm) return fail(TRA_ERR_INVALID_ARG, "plan or perm is NULL");
  if (!plan->valid) return fail(TRA_ERR_PLAN_INVALID, "the plan's last build failed");
  if (!plan->perm) return fail(TRA_ERR_INVALID_ARG, "the plan was created without regroup");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  // An asynchronous build may still run on another stream.
  if (plan->built) TRA_HIP(hipStreamWaitEvent(hs, plan->built, 0));
  TRA_HIP(hipMemcpyAsync(perm, plan->perm, plan->n_groups * tra::GROUP_SLOTS, hipMemcpyDeviceToHost, hs));
  TRA_HIP(hipStreamSynchronize(hs));
  return TRA_OK;
}

tra_status tra_plan_export_groups(const tra_plan* plan, int64_t* n_groups, int64_t* n_entries, int32_t* gptr,
                                  int32_t* glen, int32_t* glist, void* stream) {
  if (!plan) return fail(TRA_ERR_INVALID_ARG, "plan is NULL");
  if (!plan->valid) return fail(TRA_ERR_PLAN_INVALID, "the plan's last build failed");
  if (plan->shape.dtype != TRA_BF16) return fail(TRA_ERR_DTYPE, "group lists exist for bf16 plans only");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  // An asynchronous build may still run on another stream.
  if (plan->built) TRA_HIP(hipStreamWaitEvent(hs, plan->built, 0));
  TRA_HIP(hipStreamSynchronize(hs));
  if (plan->glist_stride > 0) {
    // Lists in fixed per-group slots: returned packed, in group order.
    std::vector<int32_t> len(plan->n_groups);
    TRA_HIP(hipMemcpy(len.data(), plan->glen, plan->n_groups * sizeof(int32_t), hipMemcpyDeviceToHost));
    int64_t entries = 0;
    for (int32_t l : len) entries += l;
    if (n_groups) *n_groups = plan->n_groups;
    if (n_entries) *n_entries = entries;
    if (glen) std::memcpy(glen, len.data(), len.size() * sizeof(int32_t));
    if (gptr) {
      int64_t off = 0;
      for (int64_t g = 0; g < plan->n_groups; ++g) {
        gptr[g] = static_cast<int32_t>(off);
        off += len[g];
      }
    }
    if (glist && entries > 0) {
      std::vector<int32_t> all(static_cast<size_t>(plan->n_groups) * plan->glist_stride * 2);
      TRA_HIP(hipMemcpy(all.data(), plan->glist, all.size() * sizeof(int32_t), hipMemcpyDeviceToHost));
      int64_t off = 0;
      for (int64_t g = 0; g < plan->n_groups; ++g) {
        std::memcpy(glist + 2 * off, all.data() + 2 * g * plan->glist_stride, 2 * len[g] * sizeof(int32_t));
        off += len[g];
      }
    }
    return TRA_OK;
  }
  int32_t last[2] = {0, 0};
  TRA_HIP(hipMemcpy(&last[0], plan->gptr + plan->n_groups - 1, sizeof(int32_t), hipMemcpyDeviceToHost));
  TRA_HIP(hipMemcpy(&last[1], plan->glen + plan->n_groups - 1, sizeof(int32_t), hipMemcpyDeviceToHost));
  const int64_t entries = static_cast<int64_t>(last[0]) + last[1];
  if (n_groups) *n_groups = plan->n_groups;
  if (n_entries) *n_entries = entries;
  if (gptr) TRA_HIP(hipMemcpy(gptr, plan->gptr, plan->n_groups * sizeof(int32_t), hipMemcpyDeviceToHost));
  if (glen) TRA_HIP(hipMemcpy(glen, plan->glen, plan->n_groups * sizeof(int32_t), hipMemcpyDeviceToHost));
  if (glist && entries > 0)
    TRA_HIP(hipMemcpy(glist, plan->glist, entries * 2 * sizeof(int32_t), hipMemcpyDeviceToHost));
  return TRA_OK;
}

tra_status tra_plan_stats(const tra_plan* plan, int64_t* retained, int64_t* listed, void* stream) {
  if (!plan) return fail(TRA_ERR_INVALID_ARG, "plan is NULL");
  if (!plan->valid) return fail(TRA_ERR_PLAN_INVALID, "the plan's last build failed");
  fault_arm();
  hipStream_t hs = static_cast<hipStream_t>(stream);
  // The plan's own counters and pinned words (a plan is not used by two
  // stats or drift calls at once).
  tra_plan* p = const_cast<tra_plan*>(plan);
  const tra_status cs = ensure_csr(p, hs);
  if (cs != TRA_OK) return cs;
  TRA_HIP(hipStreamWaitEvent(hs, p->built, 0));  // the latest build, on whatever stream it ran
  TRA_LAUNCH(tra::launch_clear_counters(p->counters, 2, hs));
  TRA_LAUNCH(tra::launch_stats(metric_of(plan->params), plan->lv, plan->r2, plan->shape.T, plan->row_base, plan->BH,
                               plan->tiles, plan->row_ptr, plan->col_idx, p->counters, hs));
  TRA_HIP(hipMemcpyAsync(p->totals_host + 4, p->counters, 2 * sizeof(unsigned long long), hipMemcpyDeviceToHost, hs));
  TRA_HIP(hipStreamSynchronize(hs));
  uint64_t host[2] = {static_cast<uint64_t>(p->totals_host[4]), static_cast<uint64_t>(p->totals_host[5])};
  // Pairs the attention visits under the plan's semantics: block-only masks
  // keep every pair of a listed tile pair; a vote threshold keeps the votes
  // of the listed tiles.
  if (plan->params.block_mask) host[0] = host[1];
  else if (plan->params.vote_threshold > 1) host[0] = static_cast<uint64_t>(plan->retained_votes);
  if (retained) *retained = static_cast<int64_t>(host[0]);
  if (listed) *listed = static_cast<int64_t>(host[1]);
  return TRA_OK;
}

tra_status tra_plan_drift(const tra_plan* plan, const void* q, const void* k, int64_t* changed,
                          void* stream) {
  if (!plan) return fail(TRA_ERR_INVALID_ARG, "plan is NULL");
  tra_plan* p = const_cast<tra_plan*>(plan);
  return tra::drift_with_scratch(plan, q, k, p->kbar2, p->lv2, p->counters + 2, changed, stream);
}

void tra_plan_destroy(tra_plan* plan) {
  // hipFree waits for the device's outstanding work before it releases
  // memory, so no explicit synchronisation is needed here.
  release(plan);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Reuse schedule across denoising steps.  Step policy (host side):
//   step < warmup-1                       dense attention
//   step == warmup-1, or a refresh is due dense attention + exact entropies,
//                                         plan (re)built from them
//   otherwise                             sparse attention under the plan
// A refresh is due after refresh_every sparse steps, or on the step after a
// sparse step whose tracked drift exceeded drift_threshold.  Drift tracking
// compares the pooled-key levels of the current (q, k) with those of the
// inputs the plan was built from (one pooling + entropy pass per step).
// ---------------------------------------------------------------------------
struct tra_schedule {
  tra_shape shape;
  tra_params params;
  tra_schedule_params sp;
  tra_plan* plan = nullptr;
  float* Hd = nullptr;        // dense entropies of the last re-plan step
  void* kbar = nullptr;       // pooled keys (drift tracking)
  float* Hp = nullptr;        // pooled entropies (drift tracking)
  int16_t* lv_ref = nullptr;  // pooled levels at the last re-plan
  int16_t* lv_now = nullptr;
  unsigned long long* cnt = nullptr;
  unsigned long long* cnt_host = nullptr;  // pinned
  int64_t n_queries = 0;
  int32_t step = 0, since_plan = 0;
  bool refresh_due = false;
};

namespace {

void release_schedule(tra_schedule* s) {
  if (!s) return;
  if (s->plan) release(s->plan);
  for (void* b : {static_cast<void*>(s->Hd), s->kbar, static_cast<void*>(s->Hp), static_cast<void*>(s->lv_ref),
                  static_cast<void*>(s->lv_now), static_cast<void*>(s->cnt)})
    if (b) (void)hipFree(b);
  if (s->cnt_host) (void)hipHostFree(s->cnt_host);
  delete s;
}

bool tracks_drift(const tra_schedule* s) {
  return s->sp.drift_threshold >= 0.0 && s->params.radius_override < 0.0;
}

// Pooled-key levels of (q, k) into lv (the plan's pooling geometry and table).
hipError_t pooled_levels(tra_schedule* s, const void* q, const void* k, int16_t* lv, hipStream_t hs) {
  const tra_plan* p = s->plan;
  hipError_t e = tra::launch_pool(s->shape.dtype, s->shape.head_dim, k, s->kbar, p->BH, p->pool, hs);
  if (e != hipSuccess) return e;
  const tra::EntropyArgs ea{p->params.a, p->params.c, p->params.levels_per_nat, p->table.k_lo, p->table.k_hi};
  return tra::launch_entropy(s->shape.dtype, s->shape.head_dim, q, s->kbar, p->pool_w, p->BH,
                             static_cast<int>(p->N), p->pool, ea, s->Hp, lv, hs);
}

}  // namespace

extern "C" {

tra_status tra_schedule_create(const tra_shape* shape, const tra_params* params, const tra_schedule_params* sp,
                               tra_schedule** out) {
  if (!out) return fail(TRA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!sp) return fail(TRA_ERR_INVALID_ARG, "schedule params are NULL");
  tra_status st = check_shape(shape);
  if (st != TRA_OK) return st;
  st = check_params(shape, params, nullptr);
  if (st != TRA_OK) return st;
  if (sp->warmup_steps < 1) return fail(TRA_ERR_INVALID_ARG, "warmup_steps must be >= 1");
  if (sp->refresh_every < 0) return fail(TRA_ERR_INVALID_ARG, "refresh_every must be >= 0");
  if (!std::isfinite(sp->drift_threshold)) return fail(TRA_ERR_INVALID_ARG, "drift_threshold must be finite");
  tra_schedule* s = new tra_schedule();
  s->shape = *shape;
  s->params = *params;
  s->sp = *sp;
  s->n_queries = static_cast<int64_t>(shape->B) * shape->heads * shape->T * shape->H * shape->W;
  auto fin = [&](hipError_t e) {
    release_schedule(s);
    return fail(e == hipErrorOutOfMemory ? TRA_ERR_OOM : TRA_ERR_HIP, std::string("tra_schedule_create: ") +
                                                                         hipGetErrorString(e));
  };
  fault_arm();
  hipError_t e = dev_alloc(&s->Hd, s->n_queries * sizeof(float));
  if (e != hipSuccess) return fin(e);
  if (tracks_drift(s)) {
    const tra::Grid pool = tra::make_grid(shape->T, shape->H, shape->W, params->pool_h, params->pool_w);
    const size_t kb = static_cast<size_t>(shape->B) * shape->heads * pool.count * shape->head_dim *
                      dtype_size(shape->dtype);
    if ((e = dev_alloc(&s->kbar, kb)) != hipSuccess) return fin(e);
    if ((e = dev_alloc(&s->Hp, s->n_queries * sizeof(float))) != hipSuccess) return fin(e);
    if ((e = dev_alloc(&s->lv_ref, s->n_queries * sizeof(int16_t))) != hipSuccess) return fin(e);
    if ((e = dev_alloc(&s->lv_now, s->n_queries * sizeof(int16_t))) != hipSuccess) return fin(e);
    if ((e = dev_alloc(&s->cnt, sizeof(unsigned long long))) != hipSuccess) return fin(e);
    if ((e = host_alloc(&s->cnt_host, sizeof(unsigned long long))) != hipSuccess) return fin(e);
  }
  *out = s;
  return TRA_OK;
}

tra_status tra_schedule_step(tra_schedule* s, const void* q, const void* k, const void* v, void* o, void* stream,
                             tra_step_info* info) {
  if (!s) return fail(TRA_ERR_INVALID_ARG, "schedule is NULL");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const tra_shape& sh = s->shape;
  int32_t mode;
  if (s->step < s->sp.warmup_steps - 1) {
    mode = TRA_STEP_DENSE;
  } else if (s->step == s->sp.warmup_steps - 1 || s->refresh_due ||
             (s->sp.refresh_every > 0 && s->since_plan >= s->sp.refresh_every)) {
    mode = TRA_STEP_DENSE_REPLAN;
  } else {
    mode = TRA_STEP_SPARSE;
  }
  int64_t drift = -1;
  if (mode == TRA_STEP_DENSE) {
    tra_status st = tra_dense_attention(&sh, q, k, v, o, nullptr, stream);
    if (st != TRA_OK) return st;
  } else if (mode == TRA_STEP_DENSE_REPLAN) {
    tra_status st = tra_dense_attention(&sh, q, k, v, o, s->Hd, stream);
    if (st != TRA_OK) return st;
    st = s->plan ? tra_plan_rebuild_from_entropy(s->plan, s->Hd, stream)
                 : tra_plan_create_from_entropy(&sh, &s->params, s->Hd, stream, &s->plan);
    if (st != TRA_OK) return st;
    if (tracks_drift(s)) TRA_HIP(pooled_levels(s, q, k, s->lv_ref, hs));
    s->since_plan = 0;
    s->refresh_due = false;
  } else {
    tra_status st = tra_attention(s->plan, q, k, v, o, stream);
    if (st != TRA_OK) return st;
    ++s->since_plan;
    if (tracks_drift(s)) {
      TRA_HIP(pooled_levels(s, q, k, s->lv_now, hs));
      TRA_HIP(hipMemsetAsync(s->cnt, 0, sizeof(unsigned long long), hs));
      TRA_LAUNCH(tra::launch_level_diff(s->lv_ref, s->lv_now, s->n_queries, s->cnt, hs));
      TRA_HIP(hipMemcpyAsync(s->cnt_host, s->cnt, sizeof(unsigned long long), hipMemcpyDeviceToHost, hs));
      TRA_HIP(hipStreamSynchronize(hs));
      drift = static_cast<int64_t>(*s->cnt_host);
      if (static_cast<double>(drift) > s->sp.drift_threshold * static_cast<double>(s->n_queries))
        s->refresh_due = true;
    }
  }
  if (info) {
    info->step = s->step;
    info->mode = mode;
    info->drift = drift;
  }
  ++s->step;
  return TRA_OK;
}

tra_status tra_schedule_plan(const tra_schedule* s, const tra_plan** plan) {
  if (!s || !plan) return fail(TRA_ERR_INVALID_ARG, "schedule and plan must not be NULL");
  *plan = s->plan;
  return TRA_OK;
}

void tra_schedule_destroy(tra_schedule* s) {
  // As for plans: hipFree itself waits for outstanding work.
  release_schedule(s);
}

const char* tra_status_string(tra_status s) {
  // Callers may pass any integer (ABI users, bindings); a value outside the
  // enumerators is read as an int, never as the enum.
  static_assert(sizeof(tra_status) == sizeof(int), "tra_status is int-sized");
  int v = 0;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case TRA_OK: return "TRA_OK";
    case TRA_ERR_INVALID_ARG: return "TRA_ERR_INVALID_ARG";
    case TRA_ERR_SHAPE: return "TRA_ERR_SHAPE";
    case TRA_ERR_DTYPE: return "TRA_ERR_DTYPE";
    case TRA_ERR_PLAN_MISMATCH: return "TRA_ERR_PLAN_MISMATCH";
    case TRA_ERR_OOM: return "TRA_ERR_OOM";
    case TRA_ERR_OVERFLOW: return "TRA_ERR_OVERFLOW";
    case TRA_ERR_HIP: return "TRA_ERR_HIP";
    case TRA_ERR_PLAN_INVALID: return "TRA_ERR_PLAN_INVALID";
  }
  return "TRA_ERR_UNKNOWN";
}

const char* tra_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
