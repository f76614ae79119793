// Internal declarations shared by the host API (tra_api.cpp) and the kernels
// (tra_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "tra.h"

namespace tra {

// Geometry of one head's T x H x W grid cut into th x tw rectangles per frame.
struct Grid {
  int T, H, W;
  int th, tw;     // rectangle size
  int nh, nw;     // rectangles per frame along h and w (ceil)
  int per_frame;  // nh * nw
  int count;      // T * per_frame
};

inline Grid make_grid(int T, int H, int W, int th, int tw) {
  Grid g;
  g.T = T; g.H = H; g.W = W; g.th = th; g.tw = tw;
  g.nh = (H + th - 1) / th;
  g.nw = (W + tw - 1) / tw;
  g.per_frame = g.nh * g.nw;
  g.count = T * g.per_frame;
  return g;
}

// Storage order of the pooled keys: the full rectangles of every frame first
// (frame-major, raster order inside the frame), then the rectangles cut by the
// bottom or right edge (frame-major, raster order).  The entropy kernels then
// read runs of equal-weight keys.  full_count() is the number of full ones.
__host__ __device__ inline int pool_full_count(const Grid& g) { return g.T * (g.H / g.th) * (g.W / g.tw); }
// Position of rectangle b (raster index t*per_frame + r*nw + c).
__host__ __device__ inline int pool_pos(const Grid& g, int b) {
  const int nhf = g.H / g.th, nwf = g.W / g.tw;
  const int F = nhf * nwf, G = g.per_frame - F, wr = g.nw - nwf;
  const int t = b / g.per_frame, rem = b % g.per_frame;
  const int r = rem / g.nw, c = rem % g.nw;
  if (r < nhf && c < nwf) return t * F + r * nwf + c;
  const int idx = r < nhf ? r * wr + (c - nwf) : nhf * wr + (r - nhf) * g.nw + c;
  return g.T * F + t * G + idx;
}

// Radius table on the device: the full table (n_levels x T, -1 = inactive
// frame), the largest active frame distance per level row, and a compact copy
// holding only the active entries of each row (row r at r2off[r], dmax[r] + 1
// entries) for staging in LDS.
struct RadiusTable {
  const int32_t* r2;
  const int32_t* dmax;
  const int32_t* r2c;
  const int32_t* r2off;
  int n_r2c;
  int T;
  int metric;  // METRIC_*: how the entries are compared with key distances
};

// Mask metrics.  L2: entries are squared radii of a disk per frame; L1:
// entries are L1 radii (Manhattan); WINDOW: every entry is the half-width rho
// of a window along the raster order (|n_i - n_j| <= rho).
constexpr int METRIC_L2 = 0, METRIC_L1 = 1, METRIC_WINDOW = 2;

struct EntropyArgs {
  double a, c;
  int levels_per_nat, k_lo, k_hi;
};

// Launchers (tra_kernels.hip).  All enqueue on `s` and return the launch status.
hipError_t launch_pool(int dtype, int d, const void* k, void* kbar, int BH, const Grid& pool,
                       hipStream_t s);
// kbar and pool_w in pool_pos order; pool is the pooling grid.
hipError_t launch_entropy(int dtype, int d, const void* q, const void* kbar, const float* pool_w,
                          int BH, int N, const Grid& pool, const EntropyArgs& ea, float* H_out,
                          int16_t* lv_out, hipStream_t s);
hipError_t launch_fill_levels(int16_t* lv, float* H, int64_t n, hipStream_t s);
// Tile lists: per query tile the runs of key-tile columns per (frame, tile
// row) plus the count and the frame window (csr_runs), the scan of the counts,
// and the expansion of the runs into col_idx.  DM is the largest active frame
// distance of the radius table; runs holds n_rows * (2*DM + 1) * nh int32.
// With glist, the groups' lists are filled too (fixed slots at gptr, lengths to
// glen; see launch_group_lists): in the same pass for 2 x 2 groups, by a second
// launch for 3 x 2 groups.
hipError_t launch_csr_runs(bool l1, const int16_t* lv, const RadiusTable& tab, int n_levels, int row_base,
                           int BH, const Grid& tiles, int DM, int32_t* counts, int32_t* runs, int32_t* rowwin,
                           hipStream_t s, int group_rows = 2, const int32_t* gptr = nullptr,
                           int32_t* glist = nullptr, int32_t* glen = nullptr);
hipError_t launch_scan(const int32_t* counts, int64_t n_rows, int32_t* row_ptr,
                       int64_t* totals, hipStream_t s);
hipError_t launch_csr_expand(int BH, const Grid& tiles, int DM, const int32_t* runs,
                             const int32_t* rowwin, const int32_t* row_ptr, int32_t* col_idx,
                             hipStream_t s);
// perm (bf16, may be null): per group, the order in which its queries are
// dealt to the waves (see launch_regroup); null deals the spatial half tiles.
hipError_t launch_attention(int dtype, int d, const void* q, const void* k, const void* v,
                            void* o, const int16_t* lv, const RadiusTable& tab, int row_base,
                            int BH, const Grid& tiles, const int32_t* row_ptr,
                            const int32_t* col_idx, const int32_t* gptr, const int32_t* glist,
                            const int32_t* glen, int group_rows, const uint8_t* perm, bool block_mask,
                            bool self_ref, hipStream_t s);
// Work unit of the bf16 attention kernel: a group of group_rows x 2 query
// tiles of one frame (group_rows 2 or 3, fixed per plan), run by one
// workgroup of 256 * group_rows threads (two waves per query tile).
inline int group_grid_rows(const Grid& tiles, int group_rows) { return (tiles.nh + group_rows - 1) / group_rows; }
inline int group_grid_cols(const Grid& tiles) { return (tiles.nw + 1) / 2; }
inline int64_t group_count(int BH, const Grid& tiles, int group_rows) {
  return static_cast<int64_t>(BH) * tiles.T * group_grid_rows(tiles, group_rows) * group_grid_cols(tiles);
}
// Query regrouping (groups of 2 x 2 query tiles): a group covers 16 x 16
// query positions (slot s = row * 16 + column within the group); perm +
// GROUP_SLOTS * group lists them sorted by (level, slot), positions outside
// the grid last.  Wave w of the attention kernel takes entries 32w .. 32w + 31.
constexpr int GROUP_SLOTS = 256;
hipError_t launch_regroup(const int16_t* lv, int BH, const Grid& tiles, uint8_t* perm, hipStream_t s);
// Merged tile lists of the groups, from the runs: with fill = false the length
// of each group's list to glen; with fill = true the entries (two int32 each)
// at glist + 2 * gptr[group] (gptr: exclusive scan of the lengths).  The sum
// of the lengths is at most nnz.
hipError_t launch_group_lists(bool fill, int BH, const Grid& tiles, int group_rows, int DM, const int32_t* runs,
                              const int32_t* rowwin, const int32_t* frow_ptr, const int32_t* fcol,
                              const int32_t* gptr, int32_t* glist, int32_t* glen, hipStream_t s);
// Token votes per CSR entry (votes, int16 per entry), per-row count of entries
// with at least theta votes (counts2) and the sum of their votes (added to
// *kept_votes); then the filtered CSR (row_ptr2 = scan of counts2).
// Tile lists of the 1-D window mask from per-(frame, tile row) column masks
// (tiles.nw <= 64): CSR counts (fill = false) or columns from row_ptr (fill =
// true); group lists with membership bits (count into glen, or fill from gptr).
hipError_t launch_window_csr(bool fill, const int16_t* lv, const int32_t* r2, const int32_t* dmax, int T,
                             int row_base, int BH, const Grid& tiles, const int32_t* row_ptr, int32_t* counts,
                             int32_t* col_idx, hipStream_t s);
hipError_t launch_window_groups(bool fill, const int16_t* lv, const int32_t* r2, const int32_t* dmax, int T,
                                int row_base, int BH, const Grid& tiles, int group_rows, const int32_t* gptr,
                                int32_t* glist, int32_t* glen, hipStream_t s);
hipError_t launch_votes(bool l1, const int16_t* lv, const int32_t* r2, const int32_t* dmax, int T, int row_base,
                        int BH, const Grid& tiles, const int32_t* row_ptr, const int32_t* col_idx, int theta,
                        int16_t* votes, int32_t* counts2, unsigned long long* kept_votes, hipStream_t s);
hipError_t launch_vote_compact(int64_t n_rows, const int32_t* row_ptr, const int32_t* col_idx, const int16_t* votes,
                               int theta, const int32_t* row_ptr2, int32_t* col_idx2, hipStream_t s);
// Dynamic LDS the bf16 attention kernel needs for its staged K/V buffers
// plus a compact radius table of n_r2c entries; 0 if it exceeds the device limit.
size_t attention_lds_bytes(int d, int n_r2c);

// Sets n <= 64 counters to zero (a kernel, so that callers may capture it).
hipError_t launch_clear_counters(unsigned long long* p, int n, hipStream_t s);
// Count of positions where two level arrays differ, added to *out.
hipError_t launch_level_diff(const int16_t* a, const int16_t* b, int64_t n, unsigned long long* out,
                             hipStream_t s);

// Dense warm-up pass (tra_dense.hip): O = softmax(Q K^T / sqrt(d)) V over all N
// keys of each head and, when H is not NULL, each query's exact attention
// entropy into H (fp32, B*heads*N).
hipError_t launch_dense(int dtype, int d, const void* q, const void* k, const void* v, void* o,
                        float* H, int BH, int N, hipStream_t s);
// Levels of n queries from given entropies; the entropies are copied to Hout.
hipError_t launch_levels_from_entropy(const float* Hin, int64_t n, const EntropyArgs& ea, float* Hout,
                                      int16_t* lv, hipStream_t s);

hipError_t launch_stats(int metric, const int16_t* lv, const int32_t* r2, int T, int row_base, int BH,
                        const Grid& tiles, const int32_t* row_ptr, const int32_t* col_idx,
                        unsigned long long* out2, hipStream_t s);

// Plan drift (tra_plan_drift) with its scratch in the given device memory:
// the pooled keys of k (drift_scratch_bytes' first part), the levels of (q, k)
// and one counter.  Used with the plan's own scratch and with the library's
// static scratch.
size_t drift_scratch_bytes(const tra_plan* p);
// The three parts inside drift_scratch_bytes(p) bytes at `base` (each 256-byte aligned).
void drift_scratch_layout(const tra_plan* p, unsigned char* base, void** kbar, int16_t** lv,
                          unsigned long long** counter);
inline size_t scratch_round(size_t bytes) { return (bytes + 255) & ~static_cast<size_t>(255); }
tra_status drift_with_scratch(const tra_plan* plan, const void* q, const void* k, void* kbar, int16_t* lv,
                              unsigned long long* counter, int64_t* changed, void* stream);
int plan_device(const tra_plan* p);
// Records `msg` as the calling thread's last error (tra_last_error) and returns s.
tra_status report(tra_status s, const std::string& msg);

}  // namespace tra
