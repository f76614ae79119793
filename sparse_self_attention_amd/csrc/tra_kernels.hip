// HIP kernels of the Token Radius Attention hot path for gfx950 (MI355X).
//
// Method: "Token Radius Attention for Efficient Video Generation" (summary
// page, section 2): per-query entropy -> token budget -> spatial radius that
// shrinks with temporal distance -> block-sparse tile lists -> attention over
// the listed tiles with the exact per-token disk mask.
//
// Kernels (in pipeline order):
//   pool_kernel           mean of each pool rectangle's keys, summed in fp64 and
//                         rounded once to the input dtype (HBM-bound: reads K)
//   entropy_bf16_kernel   scores against the pooled keys on bf16 matrix cores,
//                         fp32 online log-sum-exp with an entropy moment, fp64
//                         epilogue, quantised budget level (reads Q)
//   entropy_f32_kernel    the same for fp32 inputs with fp64 dot products
//   csr_runs_kernel       per query tile: union over its 64 queries of the disk
//                         footprints, as key-tile runs per frame and tile row
//   csr_expand_kernel     runs -> CSR column indices
//   window_csr_kernel,    the 1-D window generator's tile lists (raster-order
//   window_group_kernel   distance) and group lists, from per-row column masks
//   vote_kernel,          token voting: retained pairs per listed tile pair, and
//   vote_compact_kernel   the lists filtered by a vote threshold
//   group_list_kernel     runs of a group of adjacent query tiles -> their merged list
//   scan_kernel           exclusive scan of the per-tile counts
//   attn_bf16_kernel      block-sparse flash attention: S^T = K Q^T and
//                         O^T += V^T P^T on 32x32x16 bf16 MFMA, K/V tiles staged
//                         in LDS (V read back transposed with ds_read_b64_tr_b16),
//                         exact radius mask in registers, fp32 online softmax
//   attn_f32_kernel       fp32 vector variant for fp32 inputs: one query per
//                         lane, the tile's list split over the workgroup's waves
//   retained_kernel,      exact retained / listed pair counts
//   listed_kernel
//   level_diff_kernel     plan drift: queries whose level a rebuild would change
//   fill_levels_kernel    levels of the fixed-radius mode
// The dense warm-up pass (dense attention with exact entropies) is in
// tra_dense.hip.
#include "tra_internal.h"
#include "tra_device.h"

#include <math.h>

namespace tra {

// ---------------------------------------------------------------------------
// Rounding of an exact mean to the input dtype (one rounding, nearest-even).
// S is the exact sum (float64), n the count.  q = S/n is correctly rounded in
// fp64; rounding q again can only differ from rounding S/n when q falls exactly
// on a midpoint between two dtype values, and that case is decided by an exact
// comparison of |S| with midpoint*n (both exact in fp64: the midpoint has at
// most 25 significant bits and n < 2^20).
// ---------------------------------------------------------------------------
template <int SIGBITS>
__device__ double round_mean(double S, int n) {
  const double q = S / static_cast<double>(n);
  if (q == 0.0) return q;
  const double a = fabs(q);
  int e;
  const double m = frexp(a, &e);
  const double scaled = ldexp(m, SIGBITS);
  const double lo = floor(scaled);
  const double frac = scaled - lo;
  bool up;
  if (frac > 0.5) {
    up = true;
  } else if (frac < 0.5) {
    up = false;
  } else {
    const double mid = ldexp(lo + 0.5, e - SIGBITS);
    const double prod = mid * static_cast<double>(n);
    const double aS = fabs(S);
    up = aS > prod || (aS == prod && fmod(lo, 2.0) == 1.0);
  }
  return copysign(ldexp(lo + (up ? 1.0 : 0.0), e - SIGBITS), q);
}

// ---------------------------------------------------------------------------
// Key pooling.  grid (pool.count, BH), 256 threads; rectangle b is stored at
// pool_pos(b) (full rectangles first).
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(256) void pool_kernel(const void* __restrict__ k,
                                                  void* __restrict__ kbar, Grid g) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int VEC = 16 / ES;
  constexpr int NCH = D / VEC;
  constexpr int GROUPS = 256 / NCH;
  __shared__ double red[GROUPS][D];
  const int bh = blockIdx.y, b = blockIdx.x;
  const int t = b / g.per_frame, rem = b % g.per_frame;
  const int h0 = (rem / g.nw) * g.th, w0 = (rem % g.nw) * g.tw;
  const int rows = min(g.th, g.H - h0), cols = min(g.tw, g.W - w0), cnt = rows * cols;
  const int c = threadIdx.x % NCH, grp = threadIdx.x / NCH;
  const size_t N = static_cast<size_t>(g.T) * g.H * g.W;
  const char* base = static_cast<const char*>(k) + static_cast<size_t>(bh) * N * D * ES;
  double acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.0;
  for (int idx = grp; idx < cnt; idx += GROUPS) {
    const int hh = h0 + idx / cols, ww = w0 + idx % cols;
    const size_t n = (static_cast<size_t>(t) * g.H + hh) * g.W + ww;
    const uint4 raw = *reinterpret_cast<const uint4*>(base + n * D * ES + c * 16);
    const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
    if constexpr (BF16) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += static_cast<double>(__uint_as_float(wds[e] << 16));
        acc[2 * e + 1] += static_cast<double>(__uint_as_float(wds[e] & 0xffff0000u));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += static_cast<double>(__uint_as_float(wds[e]));
    }
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) red[grp][c * VEC + e] = acc[e];
  __syncthreads();
  for (int dd = threadIdx.x; dd < D; dd += 256) {
    double s = 0.0;
    for (int gi = 0; gi < GROUPS; ++gi) s += red[gi][dd];
    const size_t out = (static_cast<size_t>(bh) * g.count + pool_pos(g, b)) * D + dd;
    if constexpr (BF16) {
      const float r = static_cast<float>(round_mean<8>(s, cnt));  // exact: a bf16 value
      static_cast<uint16_t*>(kbar)[out] = static_cast<uint16_t>(__float_as_uint(r) >> 16);
    } else {
      static_cast<float*>(kbar)[out] = static_cast<float>(round_mean<24>(s, cnt));
    }
  }
}

// ---------------------------------------------------------------------------
// Entropy and budget level, shared epilogue.
//   (m, A, B) describe sum_b w_b 2^(u_b) with u = z*log2(e):
//   A = sum w 2^(u-m), B = sum w 2^(u-m) (u-m)  =>  H = ln A - ln2 * B / A.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void entropy_store(double Hd, const EntropyArgs& ea, size_t idx,
                                              float* Hout, int16_t* lvout) {
  const double L = static_cast<double>(ea.levels_per_nat) * (ea.a * Hd + ea.c);
  double kf = floor(L);
  kf = fmin(fmax(kf, static_cast<double>(ea.k_lo)), static_cast<double>(ea.k_hi));
  if (Hout) Hout[idx] = static_cast<float>(Hd);  // the entropy itself is optional (export only)
  lvout[idx] = static_cast<int16_t>(kf);
}

// bf16 inputs.  grid (ceil(N/256), BH), 256 threads: 4 waves x 64 queries,
// each wave two blocks of 32 queries (lane % 32 = query; both lanes of a
// query hold half of its pooled keys).  Pooled keys stream through LDS in
// chunks of 32 rows; each K fragment read from LDS feeds the score MFMAs of
// both query blocks.
constexpr int ENT_WAVES = 4, ENT_QB = 2, ENT_QPW = ENT_WAVES * 32 * ENT_QB;
template <int D>
__global__ __launch_bounds__(256, 3) void entropy_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kbar,
    const float* __restrict__ pool_w, int N, int NP, int NFULL, float WFULL, EntropyArgs ea,
    float* __restrict__ Hout, int16_t* __restrict__ lvout) {
  constexpr int NCH = D / 8;
  constexpr int KS = D / 16;
  __shared__ __attribute__((aligned(1024))) uint16_t kb_lds[2][32 * D];
  __shared__ __attribute__((aligned(256))) float w_lds[2][64];
  const int bh = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, col = lane & 31;
  const int n0 = blockIdx.x * ENT_QPW + wave * 32 * ENT_QB + col;  // query block qb: n0 + 32 * qb
  bf16x8 qf[ENT_QB][KS];
#pragma unroll
  for (int qb = 0; qb < ENT_QB; ++qb) {
    const uint16_t* p = q + (static_cast<size_t>(bh) * N + min(n0 + 32 * qb, N - 1)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[qb][ks] = *reinterpret_cast<const bf16x8*>(p + 16 * ks + 8 * h);
  }
  const float c1 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  float m[ENT_QB], A[ENT_QB], Bm[ENT_QB];
#pragma unroll
  for (int qb = 0; qb < ENT_QB; ++qb) {
    m[qb] = TRA_NEG_INF;
    A[qb] = 0.f;
    Bm[qb] = 0.f;
  }

  // Pooled keys stream in chunks of 32 rows (1 KB DMA segments, spread over
  // the waves; the chunk's weights through wave 0), one chunk ahead of use,
  // through range-checked buffer resources: rows past NP read as zero (weight
  // 0).  Lane l of segment s fills LDS bytes s*1KB + 16*l of the chunk, that
  // is row r and physical 16-byte chunk pc of the swizzled layout below; it
  // fetches the logical chunk pc ^ swz(r) of that row.
  constexpr int SEGS = 32 * D * 2 / 1024;  // 1 KB segments per chunk
  constexpr int SPW = (SEGS + ENT_WAVES - 1) / ENT_WAVES;
  static_assert(SEGS % ENT_WAVES == 0, "every wave streams the same number of segments");
  const i32x4 krs = make_rsrc(kbar + static_cast<size_t>(bh) * NP * D, static_cast<uint32_t>(NP * D * 2));
  const i32x4 wrs = make_rsrc(pool_w, static_cast<uint32_t>(NP * 4));
  uint32_t soff[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int sbyte = (wave + ENT_WAVES * i) * 1024 + lane * 16;
    const int srow = sbyte / (2 * D), spc = (sbyte % (2 * D)) / 16;
    soff[i] = static_cast<uint32_t>(srow * 2 * D + ((spc ^ swz<NCH>(srow)) * 16));
  }
  const uint32_t kb_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(&kb_lds[0][0])));
  const uint32_t w_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(&w_lds[0][0])));
  auto stream = [&](int ci) {
    const int b = ci & 1;
#pragma unroll
    for (int i = 0; i < SPW; ++i)
      lds_dma16_buf(krs, static_cast<uint32_t>(ci) * 32 * D * 2 + soff[i],
                    __builtin_amdgcn_readfirstlane(kb_base + b * 32 * D * 2 + (wave + ENT_WAVES * i) * 1024));
    if (wave == 0)
      lds_dma4_buf(wrs, static_cast<uint32_t>(ci) * 32 * 4 + lane * 4,
                   __builtin_amdgcn_readfirstlane(w_base + b * 64 * 4));
  };
  const int nchunks = (NP + 31) / 32;
  stream(0);
  for (int ci = 0; ci < nchunks; ++ci) {
    wait_vmcnt<0>();
    lds_barrier();
    if (ci + 1 < nchunks) stream(ci + 1);
    const uint16_t* kc = kb_lds[ci & 1];
    const float* wc = w_lds[ci & 1];
    f32x16 acc[ENT_QB];
#pragma unroll
    for (int qb = 0; qb < ENT_QB; ++qb) acc[qb] = (f32x16){0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(&kc[col * D + (((2 * ks + h) ^ swz<NCH>(col)) << 3)]);
#pragma unroll
      for (int qb = 0; qb < ENT_QB; ++qb) acc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[qb][ks], acc[qb], 0, 0, 0);
    }
    float w[16];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float4 w4 = *reinterpret_cast<const float4*>(&wc[8 * a + 4 * h]);
      w[4 * a + 0] = w4.x; w[4 * a + 1] = w4.y; w[4 * a + 2] = w4.z; w[4 * a + 3] = w4.w;
    }
    if ((ci + 1) * 32 > NP) {
      // Padded rows: weight 0 and a finite sentinel score, so that they add
      // exactly 0 to both sums (an infinite score would make 0 * inf = NaN).
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * h + (i & 3);
        if (ci * 32 + r >= NP) {
#pragma unroll
          for (int qb = 0; qb < ENT_QB; ++qb) acc[qb][i] = -3.0e38f;
        }
      }
    }
    // A chunk of full rectangles only (they come first) has one weight, which
    // then scales the chunk's two sums instead of each term.
    const bool uniform = (ci + 1) * 32 <= NFULL;
    // A lane's terms against the reference ref, unweighted in a uniform chunk.
    auto sums = [&](const f32x16& sc, float ref, float& sA, float& sB) __attribute__((always_inline)) {
      sA = 0.f;
      sB = 0.f;
      if (uniform) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float t = fmaf(sc[i], c1, -ref);
          const float e = __builtin_amdgcn_exp2f(t);
          sA += e;
          sB = fmaf(e, t, sB);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float t = fmaf(sc[i], c1, -ref);
          const float e = __builtin_amdgcn_exp2f(t) * w[i];
          sA += e;
          sB = fmaf(e, t, sB);
        }
      }
    };
    // Lazy reference: the terms are formed against the current reference;
    // only when some lane's sum leaves its bound (2^10 unweighted, 2^24
    // weighted) or is not finite, as on the first chunk (no reference yet),
    // does the wave move the reference to the exact maximum and form them
    // again.  The bounds keep every term and sum far from overflow, and a
    // reference above the chunk's scores loses nothing: it is at least the
    // largest score seen so far.
    const float bound = uniform ? 1024.f : 16777216.f;
#pragma unroll
    for (int qb = 0; qb < ENT_QB; ++qb) {
      const f32x16& sc = acc[qb];
      float sA, sB;
      sums(sc, m[qb], sA, sB);
      if (__any(!(sA <= bound))) {
        float mx = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
#pragma unroll
        for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, sc[i]), sc[i + 1]);
        mx = fmaxf(mx, sc[15]);
        // The two lane halves hold the same queries (16 keys each) and keep
        // one reference: each takes the other's chunk maximum.
        const auto mxs = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(mxs[0]), __uint_as_float(mxs[1]));
        const float mnew = fmaxf(m[qb], mx * c1);
        sums(sc, mnew, sA, sB);
        if (uniform) {
          sA *= WFULL;
          sB *= WFULL;
        }
        if (A[qb] > 0.f) {
          const float alpha = __builtin_amdgcn_exp2f(m[qb] - mnew);
          Bm[qb] = alpha * fmaf(m[qb] - mnew, A[qb], Bm[qb]) + sB;
          A[qb] = fmaf(A[qb], alpha, sA);
        } else {
          Bm[qb] = sB;
          A[qb] = sA;
        }
        m[qb] = mnew;
      } else {
        if (uniform) {
          sA *= WFULL;
          sB *= WFULL;
        }
        Bm[qb] += sB;
        A[qb] += sA;
      }
    }
  }
  // Both halves share the reference, so a query's sums are the plain sums of
  // its two halves.  Lanes 0-31 finish query block 0 and lanes 32-63 block 1:
  // one swap gives each half the other half's sums of its block.
  static_assert(ENT_QB == 2, "one query block per lane half");
  const auto As = __builtin_amdgcn_permlane32_swap(__float_as_uint(A[0]), __float_as_uint(A[1]), false, false);
  const auto Bs = __builtin_amdgcn_permlane32_swap(__float_as_uint(Bm[0]), __float_as_uint(Bm[1]), false, false);
  const int n = n0 + 32 * h;
  if (n < N) {
    const double At = static_cast<double>(__uint_as_float(As[0])) + static_cast<double>(__uint_as_float(As[1]));
    const double Bt = static_cast<double>(__uint_as_float(Bs[0])) + static_cast<double>(__uint_as_float(Bs[1]));
    const double Hd = log(At) - 0.6931471805599453 * Bt / At;
    entropy_store(Hd, ea, static_cast<size_t>(bh) * N + n, Hout, lvout);
  }
}

// fp32 inputs: one thread per query, fp64 dot products (exact products of two
// fp32 values) and fp64 online log-sum-exp.  grid (ceil(N/256), BH).
template <int D>
__global__ __launch_bounds__(256) void entropy_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kbar, const float* __restrict__ pool_w,
    int N, int NP, EntropyArgs ea, float* __restrict__ Hout, int16_t* __restrict__ lvout) {
  __shared__ float kb_lds[32][D];
  __shared__ float w_lds[32];
  const int bh = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  const float* qp = q + (static_cast<size_t>(bh) * N + min(n, N - 1)) * D;
  float qr[D];
#pragma unroll
  for (int dd = 0; dd < D; dd += 4) {
    const float4 v = *reinterpret_cast<const float4*>(qp + dd);
    qr[dd] = v.x; qr[dd + 1] = v.y; qr[dd + 2] = v.z; qr[dd + 3] = v.w;
  }
  const float* kb = kbar + static_cast<size_t>(bh) * NP * D;
  const double inv_sqrt_d = 1.0 / sqrt(static_cast<double>(D));
  double m = -__builtin_inf(), A = 0.0, Bm = 0.0;  // natural-log units
  for (int base = 0; base < NP; base += 32) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < 32 * D; idx += 256) {
      const int r = idx / D, c = idx % D;
      kb_lds[r][c] = base + r < NP ? kb[static_cast<size_t>(base + r) * D + c] : 0.f;
    }
    if (threadIdx.x < 32) w_lds[threadIdx.x] = base + threadIdx.x < NP ? pool_w[base + threadIdx.x] : 0.f;
    __syncthreads();
    const int rows = min(32, NP - base);
    for (int r = 0; r < rows; ++r) {
      double z = 0.0;
#pragma unroll
      for (int dd = 0; dd < D; ++dd) z = fma(static_cast<double>(qr[dd]), static_cast<double>(kb_lds[r][dd]), z);
      z *= inv_sqrt_d;
      const double w = w_lds[r];
      if (z > m) {
        const double alpha = A > 0.0 ? exp(m - z) : 0.0;
        Bm = A > 0.0 ? alpha * (Bm + (m - z) * A) : 0.0;
        A *= alpha;
        m = z;
      }
      const double t = z - m, e = w * exp(t);
      A += e;
      Bm += e * t;
    }
  }
  if (n < N) entropy_store(log(A) - Bm / A, ea, static_cast<size_t>(bh) * N + n, Hout, lvout);
}

__global__ void fill_levels_kernel(int16_t* lv, float* H, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) {
    lv[i] = -1;
    H[i] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// Tile lists.
//
// Step 1 (csr_runs_kernel): one wave per query tile, lane = query (tile-local
// row-major).  For every key frame within the wave's largest active temporal
// distance and every key-tile row the disks reach, a query's footprint is the
// column interval [w - a, w + a], a = isqrt(R2 - dh^2), as a run of key-tile
// columns that contains the query tile's own column; the union over the wave
// is therefore the run [min lo, max hi].  The kernel writes the row's count,
// its frame window (first frame | frames << 16) and the runs
// (LO | HI << 16, empty = HI < LO) at runs + row * RS, RS = (2*DM + 1) * nh,
// frame-major, tile rows in order.  grid (ceil(tiles.count/4), BH).
// Step 2: scan of the counts (scan_kernel).
// Step 3 (csr_expand_kernel): one wave per row expands the runs into col_idx.
// ---------------------------------------------------------------------------
constexpr int32_t RUN_EMPTY = 0xffff;  // LO = 0xffff, HI = 0

// Distance metric of the mask.  Euclidean (L1 = false): a table entry is a
// squared radius and key (dh, dw) is kept iff dh^2 + dw^2 <= entry.
// Manhattan (L1 = true): the entry is an L1 radius and the test is
// |dh| + |dw| <= entry.
// Largest |dh| with a kept key, for an entry thr >= 0.
template <bool L1>
__device__ __forceinline__ int mask_reach(int thr) {
  return L1 ? thr : isqrt_i(thr);
}
// Half-width of the kept columns at row offset dh (-1: none), thr >= 0.
template <bool L1>
__device__ __forceinline__ int mask_half_width(int thr, int dh) {
  if (L1) {
    const int a = thr - abs(dh);
    return a >= 0 ? a : -1;
  }
  const int rem = thr - dh * dh;
  return rem >= 0 ? isqrt_i(rem) : -1;
}

// One wave per query tile (8 x 8 tiles: 64 queries).  The wave's eight groups
// of 8 lanes take eight (temporal distance, key-tile row) pairs at a time; in
// a pair, lane c folds the 8 queries of tile column c, and one reduction over
// the group's 8 lanes gives the run.  A column's queries share their center
// w, so their intervals [w - a, w + a] are nested and the widest decides: the
// lane takes the largest R2 - dh^2 (L1: R - |dh|) and one square root.  The
// radius table is staged in LDS (dynamic): per level row its largest active
// distance and the offset of its active entries in the compact table, then
// the compact table itself.
template <bool FILL, int GR>
__device__ __forceinline__ void group_fill(Grid g, int DM, int ngh, int ngw, int64_t gid, int lane,
                                           const int32_t* __restrict__ runs, const int32_t* __restrict__ rowwin,
                                           const int32_t* __restrict__ frow_ptr, const int32_t* __restrict__ fcol,
                                           const int32_t* __restrict__ gptr, int2* __restrict__ glist,
                                           int32_t* __restrict__ glen);

// GR = 2: a workgroup of 2 * GR waves takes the GR x 2 query tiles of one
// group of the bf16 attention kernel (wave m: tile row m / 2, column m % 2 of
// the group; grid (groups per head, BH)), and once the runs of its tiles are
// written wave 0 merges them into the group's list at gptr[group]
// (group_fill), so that no second pass reads the runs back.  GR = 0: four
// waves, one query tile each (grid (ceil(tiles per head / 4), BH)).
template <bool L1, int GR>
__global__ __launch_bounds__(256) void csr_runs_kernel(const int16_t* __restrict__ lv,
                                                      const int32_t* __restrict__ r2c,
                                                      const int32_t* __restrict__ r2off,
                                                      const int32_t* __restrict__ dmax, int n_levels,
                                                      int n_r2c, int T,
                                                      int row_base, Grid g, int tw_shift, int DM,
                                                      int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ runs,
                                                      int32_t* __restrict__ rowwin, int ngh, int ngw,
                                                      const int32_t* __restrict__ gptr,
                                                      int2* __restrict__ glist, int32_t* __restrict__ glen) {
  static_assert(GR == 0 || GR == 2, "four waves: one query tile each, or the four tiles of a 2 x 2 group");
  constexpr bool GROUPS = GR > 0;
  constexpr int NT = 256;
  extern __shared__ int32_t tab_s[];
  int32_t* dmax_s = tab_s;
  int32_t* off_s = tab_s + n_levels;
  int32_t* r2c_s = tab_s + 2 * n_levels;
  for (int i = threadIdx.x; i < n_levels; i += NT) {
    dmax_s[i] = dmax[i];
    off_s[i] = r2off[i];
  }
  for (int i = threadIdx.x; i < n_r2c; i += NT) r2c_s[i] = r2c[i];
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bh = blockIdx.y;
  int tile;
  bool valid;
  if constexpr (GROUPS) {
    const int grem = blockIdx.x;  // group within the head
    const int gc = grem % ngw, gr = (grem / ngw) % ngh, tg = grem / (ngw * ngh);
    const int tr = gr * GR + (wave >> 1), tc = 2 * gc + (wave & 1);
    valid = tr < g.nh && tc < g.nw;
    tile = (tg * g.nh + tr) * g.nw + tc;
  } else {
    tile = blockIdx.x * 4 + wave;
    valid = tile < g.count;
  }
  if (valid) {  // wave-uniform
  const size_t N = static_cast<size_t>(g.T) * g.H * g.W;
  const int64_t row = static_cast<int64_t>(bh) * g.count + tile;
  const int tq = tile / g.per_frame, rem = tile % g.per_frame;
  const int h0 = (rem / g.nw) * g.th, w0 = (rem % g.nw) * g.tw;
  // Lane 8*grp + c takes column c of the tile (its 8 queries, one per tile
  // row) in pair group grp: table offset and largest active distance per row
  // (dm = -1 for positions outside the grid).
  const int c = lane & 7, grp = lane >> 3;
  const int wl = w0 + c;
  int toff[8], dm[8];
  int dmx = -1;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    toff[r] = 0;
    dm[r] = -1;
    if (h0 + r < g.H && wl < g.W) {
      const int trow =
          lv[static_cast<size_t>(bh) * N + (static_cast<size_t>(tq) * g.H + h0 + r) * g.W + wl] - row_base;
      toff[r] = off_s[trow];
      dm[r] = dmax_s[trow];
    }
    dmx = max(dmx, dm[r]);
  }
  const int dmw = wave_max_u(dmx);
  const int t_lo = max(0, tq - dmw), t_hi = min(T - 1, tq + dmw);
  int32_t* rrow = runs + row * static_cast<int64_t>((2 * DM + 1) * g.nh);
  int count = 0;
  // Pairs (delta, key-tile row), delta-major; frames tq - delta and tq +
  // delta see the same disks, so each pair's run is written for both.  The
  // eight lane groups take eight pairs per step: pair p = p0 + grp, with
  // (delta, tr) advanced incrementally.
  const int npairs = (dmw + 1) * g.nh;
  int delta = grp / g.nh, tr = grp % g.nh;
  for (int p0 = 0; p0 < npairs; p0 += 8) {
    const bool live = p0 + grp < npairs;
    const int r0 = tr * g.th, r1 = min(g.H, r0 + g.th) - 1;
    // The column's 8 queries share its center, so their intervals are nested
    // and the widest decides: the largest R2 - dh^2 (L1: R - |dh|) at the
    // nearest key row of the tile row, then one square root.  (The table
    // reads are in bounds for every lane and issued together; `live` only
    // masks the result.)
    int vt[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) vt[r] = r2c_s[toff[r] + min(delta, max(dm[r], 0))];
    int best = -1;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int hq = h0 + r;
      const int dh = max(0, max(r0 - hq, hq - r1));
      const int w2 = L1 ? vt[r] - dh : vt[r] - dh * dh;
      best = max(best, delta <= dm[r] ? w2 : -1);
    }
    const int a = (live && best >= 0) ? mask_reach<L1>(best) : -1;
    int lo = 0x7fffffff, hi = -1;
    if (a >= 0) {
      lo = max(0, wl - a) >> tw_shift;
      hi = min(g.W - 1, wl + a) >> tw_shift;
    }
    // Min / max over the 8 lanes of the group: within quads, then across the
    // two quads of each half row (row_half_mirror pairs lane i with 7 - i).
    lo = min(lo, __builtin_amdgcn_update_dpp(0, lo, 0xB1, 0xF, 0xF, false));
    hi = max(hi, __builtin_amdgcn_update_dpp(0, hi, 0xB1, 0xF, 0xF, false));
    lo = min(lo, __builtin_amdgcn_update_dpp(0, lo, 0x4E, 0xF, 0xF, false));
    hi = max(hi, __builtin_amdgcn_update_dpp(0, hi, 0x4E, 0xF, 0xF, false));
    lo = min(lo, __builtin_amdgcn_update_dpp(0, lo, 0x141, 0xF, 0xF, false));
    hi = max(hi, __builtin_amdgcn_update_dpp(0, hi, 0x141, 0xF, 0xF, false));
    if (live && c == 0) {
      const bool below = tq - delta >= 0, above = delta > 0 && tq + delta <= T - 1;
      const int32_t run = hi >= lo ? (lo | (hi << 16)) : RUN_EMPTY;
      if (hi >= lo) count += (hi - lo + 1) * ((below ? 1 : 0) + (above ? 1 : 0));
      if (below) rrow[(tq - delta - t_lo) * g.nh + tr] = run;
      if (above) rrow[(tq + delta - t_lo) * g.nh + tr] = run;
    }
    tr += 8;
    while (tr >= g.nh) {
      tr -= g.nh;
      ++delta;
    }
  }
  count = wave_sum_u(count);
  if (lane == 0) {
    counts[row] = count;
    rowwin[row] = t_lo | (max(0, t_hi - t_lo + 1) << 16);
  }
  }
  if constexpr (GROUPS) {
    __syncthreads();  // the group's runs and windows, written above, are visible to wave 0
    if (wave == 0)
      group_fill<true, GR>(g, DM, ngh, ngw, static_cast<int64_t>(bh) * g.T * ngh * ngw + blockIdx.x, lane, runs,
                           rowwin, nullptr, nullptr, gptr, glist, glen);
  }
}

// Step 3: expand the runs of each row into col_idx (ascending tile index).
// One wave per row, runs taken 64 at a time.
__global__ __launch_bounds__(256) void csr_expand_kernel(Grid g, int DM, int64_t n_rows,
                                                        const int32_t* __restrict__ runs,
                                                        const int32_t* __restrict__ rowwin,
                                                        const int32_t* __restrict__ row_ptr,
                                                        int32_t* __restrict__ col_idx) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;  // wave-uniform
  const int32_t* rrow = runs + row * static_cast<int64_t>((2 * DM + 1) * g.nh);
  const int win = rowwin[row];
  const int t_lo = win & 0xffff, nruns = (win >> 16) * g.nh;
  int out = row_ptr[row];
  for (int j0 = 0; j0 < nruns; j0 += 64) {
    const int j = j0 + lane;
    const int run = j < nruns ? rrow[j] : RUN_EMPTY;
    const int LO = run & 0xffff, HI = run >> 16;
    const int len = HI >= LO ? HI - LO + 1 : 0;
    int total;
    const int excl = wave_excl_scan(len, lane, &total);
    const int base = ((t_lo + j / g.nh) * g.nh + j % g.nh) * g.nw + LO;
    for (int c = 0; c < len; ++c) col_idx[out + excl + c] = base + c;
    out += total;
  }
}

// Sorted-array membership (binary search).
__device__ __forceinline__ bool sorted_contains(const int32_t* __restrict__ a, int n, int key) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < key) lo = mid + 1;
    else hi = mid;
  }
  return lo < n && a[lo] == key;
}

// Union of the tile lists of a group of GR x 2 query tiles of one
// frame (the unit of work of the bf16 attention kernel), from the runs of
// their rows: per (frame, tile row) the union of the runs is again a run
// (each nonempty run contains its own query tile's column, and the group's
// columns are adjacent).  Entries in ascending order as
// (frame | member << 16 | ragged << 31, row0 | col0 << 16): member has bit
// m = 2 * (tile row in the group) + (tile column in the group) set when query
// tile m lists the key tile, ragged marks a tile cut by the bottom or right
// edge of the grid.  With a vote threshold above one (frow_ptr != NULL) a
// query tile lists a key tile when its filtered CSR row holds it, and key
// tiles no query tile lists are left out.  FILL = false: the list's length to
// glen[gid]; FILL = true: the entries from glist + gptr[gid].  One wave per
// group.
template <bool FILL, int GR>
__device__ __forceinline__ void group_fill(Grid g, int DM, int ngh, int ngw, int64_t gid, int lane,
                                           const int32_t* __restrict__ runs, const int32_t* __restrict__ rowwin,
                                           const int32_t* __restrict__ frow_ptr, const int32_t* __restrict__ fcol,
                                           const int32_t* __restrict__ gptr, int2* __restrict__ glist,
                                           int32_t* __restrict__ glen) {
  const int64_t per_head = static_cast<int64_t>(g.T) * ngh * ngw;
  const int64_t bh = gid / per_head;
  const int grem = static_cast<int>(gid % per_head);
  const int gc = grem % ngw, gr = (grem / ngw) % ngh, tq = grem / (ngw * ngh);
  const int64_t RS = static_cast<int64_t>((2 * DM + 1) * g.nh);
  constexpr int NR = 2 * GR;
  int64_t rows[NR];
  int wlo[NR], wn[NR];
  int t_lo = 0x7fffffff, t_hi = -1;
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    const int tr = gr * GR + (m >> 1), tc = 2 * gc + (m & 1);
    rows[m] = bh * g.count + (static_cast<int64_t>(tq) * g.nh + tr) * g.nw + tc;
    const int w = (tr < g.nh && tc < g.nw) ? rowwin[rows[m]] : 0;
    wlo[m] = w & 0xffff;
    wn[m] = w >> 16;
    if (wn[m] > 0) {
      t_lo = min(t_lo, wlo[m]);
      t_hi = max(t_hi, wlo[m] + wn[m] - 1);
    }
  }
  const int nruns = t_hi >= t_lo ? (t_hi - t_lo + 1) * g.nh : 0;
  int64_t out = FILL ? gptr[gid] : 0;
  const int64_t beg = out;
  for (int j0 = 0; j0 < nruns; j0 += 64) {
    const int j = j0 + lane;
    const int tk = t_lo + j / g.nh, ktr = j % g.nh;
    int LO = 0xffff, HI = 0;
    int rlo[NR], rhi[NR];
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      rlo[m] = 0xffff;
      rhi[m] = 0;
      if (j < nruns && tk >= wlo[m] && tk < wlo[m] + wn[m]) {
        const int r = runs[rows[m] * RS + (tk - wlo[m]) * g.nh + ktr];
        rlo[m] = r & 0xffff;
        rhi[m] = r >> 16;
        LO = min(LO, rlo[m]);
        HI = max(HI, rhi[m]);
      }
    }
    const int base = (tk * g.nh + ktr) * g.nw;
    auto member = [&](int c) {
      int mb = 0;
#pragma unroll
      for (int m = 0; m < NR; ++m) {
        bool in = c >= rlo[m] && c <= rhi[m];
        if (in && frow_ptr) {
          const int b0 = frow_ptr[rows[m]];
          in = sorted_contains(fcol + b0, frow_ptr[rows[m] + 1] - b0, base + c);
        }
        mb |= in ? 1 << m : 0;
      }
      return mb;
    };
    int len = 0;
    if (frow_ptr) {
      for (int c = LO; c <= HI; ++c) len += member(c) != 0;
    } else {
      len = HI >= LO ? HI - LO + 1 : 0;
    }
    int total;
    const int excl = wave_excl_scan(len, lane, &total);
    if (FILL) {
      const int kr0 = ktr * g.th;
      const bool row_cut = kr0 + g.th > g.H;
      int o = 0;
      for (int c = LO; c <= HI; ++c) {
        const int mb = member(c);
        if (mb == 0) continue;
        const int kc0 = c * g.tw;
        const bool ragged = row_cut || kc0 + g.tw > g.W;
        glist[out + excl + o] = make_int2(tk | (mb << 16) | (ragged ? static_cast<int>(0x80000000u) : 0),
                                          kr0 | (kc0 << 16));
        ++o;
      }
    }
    out += total;
  }
  if (lane == 0) glen[gid] = static_cast<int32_t>(out - beg);
}

template <bool FILL, int GR>
__global__ __launch_bounds__(256) void group_list_kernel(Grid g, int DM, int ngh, int ngw, int64_t n_groups,
                                                        const int32_t* __restrict__ runs,
                                                        const int32_t* __restrict__ rowwin,
                                                        const int32_t* __restrict__ frow_ptr,
                                                        const int32_t* __restrict__ fcol,
                                                        const int32_t* __restrict__ gptr,
                                                        int2* __restrict__ glist, int32_t* __restrict__ glen) {
  const int lane = threadIdx.x & 63;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (gid >= n_groups) return;  // wave-uniform
  group_fill<FILL, GR>(g, DM, ngh, ngw, gid, lane, runs, rowwin, frow_ptr, fcol, gptr, glist, glen);
}

// Token votes of every tile-list entry: one wave per query tile (lane =
// query), each lane counting the keys of the entry's key tile it retains.
// votes[e] receives the entry's total; counts2[row] the number of entries with
// at least theta votes, and *kept_votes the sum of their votes (the retained
// pairs under the threshold).
template <bool L1>
__global__ __launch_bounds__(256) void vote_kernel(const int16_t* __restrict__ lv, const int32_t* __restrict__ r2,
                                                  const int32_t* __restrict__ dmax, int T, int row_base, Grid g,
                                                  int64_t n_rows, const int32_t* __restrict__ row_ptr,
                                                  const int32_t* __restrict__ col_idx, int theta,
                                                  int16_t* __restrict__ votes, int32_t* __restrict__ counts2,
                                                  unsigned long long* __restrict__ kept_votes) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;  // wave-uniform
  const int bh = static_cast<int>(row / g.count), tile = static_cast<int>(row % g.count);
  const size_t N = static_cast<size_t>(g.T) * g.H * g.W;
  const int tq = tile / g.per_frame, rem = tile % g.per_frame;
  const int hq = (rem / g.nw) * g.th + (lane >> 3), wq = (rem % g.nw) * g.tw + (lane & 7);
  const bool valid = hq < g.H && wq < g.W;
  int trow = 0, dm = -1;
  if (valid) {
    trow = lv[static_cast<size_t>(bh) * N + (static_cast<size_t>(tq) * g.H + hq) * g.W + wq] - row_base;
    dm = dmax[trow];
  }
  int kept = 0;
  unsigned long long kv = 0;
  // Entries come in runs of one (frame, key tile row): the lane's chord
  // half-widths over the tile row's 8 key rows (-1: none) are computed once
  // per run.
  int half[8];
  int prevK = -2, kcol = 0;
  for (int e = row_ptr[row]; e < row_ptr[row + 1]; ++e) {
    const int K = col_idx[e];
    // The next column of the same run needs no division (wave-uniform test).
    if (K == prevK + 1 && kcol + 1 < g.nw) {
      ++kcol;
    } else {
      const int tk = K / g.per_frame, krem = K % g.per_frame;
      const int ktr = krem / g.nw;
      kcol = krem % g.nw;
      const int kr0 = ktr * g.th;
      const int delta = tk > tq ? tk - tq : tq - tk;
      const int thr = (valid && delta <= dm) ? r2[trow * T + delta] : -1;
#pragma unroll
      for (int r = 0; r < 8; ++r)
        half[r] = (thr >= 0 && kr0 + r < g.H) ? mask_half_width<L1>(thr, kr0 + r - hq) : -1;
    }
    prevK = K;
    const int kc0 = kcol * g.tw;
    const int kc1 = min(kc0 + g.tw, g.W) - 1;
    int v = 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int a = half[r];
      if (a >= 0) v += max(0, min(wq + a, kc1) - max(wq - a, kc0) + 1);
    }
    v = wave_sum_u(v);
    if (lane == 0) votes[e] = static_cast<int16_t>(v);
    if (v >= theta) {
      ++kept;
      kv += static_cast<unsigned long long>(v);
    }
  }
  if (lane == 0) {
    counts2[row] = kept;
    atomicAdd(kept_votes, kv);
  }
}

// Entries with at least theta votes, in order, into the filtered CSR.  One
// wave per row.
__global__ __launch_bounds__(256) void vote_compact_kernel(int64_t n_rows, const int32_t* __restrict__ row_ptr,
                                                          const int32_t* __restrict__ col_idx,
                                                          const int16_t* __restrict__ votes, int theta,
                                                          const int32_t* __restrict__ row_ptr2,
                                                          int32_t* __restrict__ col_idx2) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;  // wave-uniform
  const int b = row_ptr[row], e = row_ptr[row + 1];
  int out = row_ptr2[row];
  for (int j0 = b; j0 < e; j0 += 64) {
    const int j = j0 + lane;
    const int keep = (j < e && votes[j] >= theta) ? 1 : 0;
    int total;
    const int excl = wave_excl_scan(keep, lane, &total);
    if (keep) col_idx2[out + excl] = col_idx[j];
    out += total;
  }
}

// ---------------------------------------------------------------------------
// Tile lists of the 1-D window mask (key j kept iff |n_i - n_j| <= rho along
// the raster order).  A query's window touches, in one key tile row of one
// frame, a prefix, a middle run and/or a suffix of the tile columns, so the
// lists are built from 64-bit column masks (at most 64 tile columns).
// ---------------------------------------------------------------------------
// Tile columns of (frame tk, tile row ktr) that the head-local raster range
// [lo, hi] touches.
__device__ __forceinline__ uint64_t window_tile_mask(int lo, int hi, int tk, int ktr, const Grid& g) {
  const int F = tk * g.H * g.W;
  const int r0 = ktr * g.th, r1 = min(r0 + g.th, g.H) - 1;
  const int a = max(lo - F, r0 * g.W), b = min(hi - F, r1 * g.W + g.W - 1);
  if (a > b) return 0;
  const int ra = a / g.W, rb = b / g.W;
  const int ca = a - ra * g.W, cb = b - rb * g.W;
  auto cols = [&](int c0, int c1) {
    const int t0 = c0 / g.tw, t1 = c1 / g.tw;
    return ((2ull << t1) - 1ull) & ~((1ull << t0) - 1ull);
  };
  if (ra == rb) return cols(ca, cb);
  if (rb > ra + 1) return cols(0, g.W - 1);
  return cols(ca, g.W - 1) | cols(0, cb);
}

// Per query lane: the window [lo, hi] (lo > hi when the query is outside the
// grid) and the largest frame distance it reaches.
struct WindowQuery {
  int lo, hi, dm;
};
__device__ __forceinline__ WindowQuery window_query(const int16_t* __restrict__ lv, const int32_t* __restrict__ r2,
                                                    const int32_t* __restrict__ dmax, int T, int row_base,
                                                    const Grid& g, int bh, int tq, int hq, int wq) {
  WindowQuery w{1, 0, -1};
  if (hq < g.H && wq < g.W) {
    const int N = g.T * g.H * g.W;
    const int n = (tq * g.H + hq) * g.W + wq;
    const int trow = lv[static_cast<size_t>(bh) * N + n] - row_base;
    const int rho = r2[trow * T];
    w.lo = max(0, n - rho);
    w.hi = min(N - 1, n + rho);
    w.dm = dmax[trow];
  }
  return w;
}

// CSR rows: FILL = false writes each row's count, FILL = true its key tiles
// from row_ptr[row] on.  One wave per query tile, lane = query.
template <bool FILL>
__global__ __launch_bounds__(256) void window_csr_kernel(const int16_t* __restrict__ lv, const int32_t* __restrict__ r2,
                                                        const int32_t* __restrict__ dmax, int T, int row_base, Grid g,
                                                        int64_t n_rows, const int32_t* __restrict__ row_ptr,
                                                        int32_t* __restrict__ counts, int32_t* __restrict__ col_idx) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;  // wave-uniform
  const int bh = static_cast<int>(row / g.count), tile = static_cast<int>(row % g.count);
  const int tq = tile / g.per_frame, rem = tile % g.per_frame;
  const WindowQuery wq = window_query(lv, r2, dmax, T, row_base, g, bh, tq, (rem / g.nw) * g.th + (lane >> 3),
                                     (rem % g.nw) * g.tw + (lane & 7));
  const int dmw = wave_max_u(wq.dm);
  const int t_lo = max(0, tq - dmw), t_hi = min(T - 1, tq + dmw);
  int out = FILL ? row_ptr[row] : 0;
  for (int tk = t_lo; tk <= t_hi; ++tk) {
    for (int ktr = 0; ktr < g.nh; ++ktr) {
      const uint64_t M = wave_or_u64(window_tile_mask(wq.lo, wq.hi, tk, ktr, g));
      if (FILL && lane < g.nw && ((M >> lane) & 1ull))
        col_idx[out + __popcll(M & ((1ull << lane) - 1ull))] = (tk * g.nh + ktr) * g.nw + lane;
      out += __popcll(M);
    }
  }
  if (!FILL && lane == 0) counts[row] = out;
}

// Query regrouping by level: one workgroup of GROUP_SLOTS threads per group
// of 2 x 2 query tiles sorts the keys (level << 8 | slot) of the group's positions
// (slot = row * 16 + column inside the group; positions outside the grid get
// the largest level) with a bitonic network in LDS and stores the sorted
// slots.  The keys are distinct, so the order is deterministic.
__global__ __launch_bounds__(GROUP_SLOTS) void regroup_kernel(const int16_t* __restrict__ lv, Grid g, int ngh,
                                                             int ngw, uint8_t* __restrict__ perm) {
  __shared__ uint32_t key[GROUP_SLOTS];
  const int64_t gid = blockIdx.x;
  const int per_head = g.T * ngh * ngw;
  const int bh = static_cast<int>(gid / per_head), grem = static_cast<int>(gid % per_head);
  const int tq = grem / (ngh * ngw), gr = (grem % (ngh * ngw)) / ngw, gc = grem % ngw;
  const int s = threadIdx.x;
  const int hq = gr * 16 + (s >> 4), wq = gc * 16 + (s & 15);
  const size_t N = static_cast<size_t>(g.T) * g.H * g.W;
  const uint32_t level = (hq < g.H && wq < g.W)
                             ? static_cast<uint32_t>(lv[static_cast<size_t>(bh) * N + (static_cast<size_t>(tq) * g.H + hq) * g.W + wq] + 32768)
                             : 0xffffu;
  key[s] = (level << 8) | static_cast<uint32_t>(s);
  __syncthreads();
  for (int kk = 2; kk <= GROUP_SLOTS; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      const int p = s ^ j;
      if (p > s) {
        const uint32_t a = key[s], b = key[p];
        if ((a > b) == ((s & kk) == 0)) {
          key[s] = b;
          key[p] = a;
        }
      }
      __syncthreads();
    }
  }
  perm[gid * GROUP_SLOTS + s] = static_cast<uint8_t>(key[s] & 0xffu);
}

// Group lists (GR x 2 query tiles, the entries and membership bits of
// group_list_kernel).  One wave per group.
template <bool FILL, int GR>
__global__ __launch_bounds__(256) void window_group_kernel(const int16_t* __restrict__ lv, const int32_t* __restrict__ r2,
                                                          const int32_t* __restrict__ dmax, int T, int row_base, Grid g,
                                                          int ngh, int ngw, int64_t n_groups,
                                                          const int32_t* __restrict__ gptr, int2* __restrict__ glist,
                                                          int32_t* __restrict__ glen) {
  const int lane = threadIdx.x & 63;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (gid >= n_groups) return;  // wave-uniform
  const int64_t per_head = static_cast<int64_t>(g.T) * ngh * ngw;
  const int bh = static_cast<int>(gid / per_head);
  const int grem = static_cast<int>(gid % per_head);
  const int gc = grem % ngw, gr = (grem / ngw) % ngh, tq = grem / (ngw * ngh);
  constexpr int NR = 2 * GR;
  WindowQuery wq[NR];
  int dm = -1;
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    const int tr = gr * GR + (m >> 1), tc = 2 * gc + (m & 1);
    wq[m] = WindowQuery{1, 0, -1};
    if (tr < g.nh && tc < g.nw)
      wq[m] = window_query(lv, r2, dmax, T, row_base, g, bh, tq, tr * g.th + (lane >> 3), tc * g.tw + (lane & 7));
    dm = max(dm, wq[m].dm);
  }
  const int dmw = wave_max_u(dm);
  const int t_lo = max(0, tq - dmw), t_hi = min(T - 1, tq + dmw);
  int64_t out = FILL ? gptr[gid] : 0;
  const int64_t beg = out;
  for (int tk = t_lo; tk <= t_hi; ++tk) {
    for (int ktr = 0; ktr < g.nh; ++ktr) {
      uint64_t M[NR], U = 0;
#pragma unroll
      for (int m = 0; m < NR; ++m) {
        M[m] = wave_or_u64(window_tile_mask(wq[m].lo, wq[m].hi, tk, ktr, g));
        U |= M[m];
      }
      if (FILL && lane < g.nw && ((U >> lane) & 1ull)) {
        int mb = 0;
#pragma unroll
        for (int m = 0; m < NR; ++m) mb |= ((M[m] >> lane) & 1ull) ? 1 << m : 0;
        const int kr0 = ktr * g.th, kc0 = lane * g.tw;
        const bool ragged = kr0 + g.th > g.H || kc0 + g.tw > g.W;
        glist[out + __popcll(U & ((1ull << lane) - 1ull))] =
            make_int2(tk | (mb << 16) | (ragged ? static_cast<int>(0x80000000u) : 0), kr0 | (kc0 << 16));
      }
      out += __popcll(U);
    }
  }
  if (lane == 0) glen[gid] = static_cast<int32_t>(out - beg);
}

// Exclusive scan of per-row counts.  One workgroup of 1024 threads walks the
// counts in tiles of 4096 (4 per thread, 16-byte loads): a thread's partial
// sums, a wave scan of the thread totals, a scan of the 16 wave totals, and a
// 64-bit carry across tiles.  totals[0] = nnz, totals[1] = longest row,
// totals[2] = 1 if nnz >= 2^31 (row_ptr then holds wrapped values).
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ counts,
                                                   int64_t n, int32_t* __restrict__ row_ptr,
                                                   int64_t* __restrict__ totals) {
  __shared__ long long wsum[16];
  __shared__ int wmax[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  long long carry = 0;
  int mx = 0;
  for (int64_t base = 0; base < n; base += 4096) {
    const int64_t i0 = base + 4 * tid;
    int c[4];
    if (i0 + 3 < n && (reinterpret_cast<uintptr_t>(counts + i0) & 15) == 0) {
      const int4 v = *reinterpret_cast<const int4*>(counts + i0);
      c[0] = v.x; c[1] = v.y; c[2] = v.z; c[3] = v.w;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) c[k] = i0 + k < n ? counts[i0 + k] : 0;
    }
    const int t = c[0] + c[1] + c[2] + c[3];
    mx = max(mx, max(max(c[0], c[1]), max(c[2], c[3])));
    // Inclusive wave scan of the thread totals (64-bit: a tile can exceed 2^31).
    long long x = t;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    long long wpre = 0, tile = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const long long ws = wsum[w];
      wpre += w < wave ? ws : 0;
      tile += ws;
    }
    long long run = carry + wpre + (x - t);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (i0 + k < n) row_ptr[i0 + k] = static_cast<int32_t>(run);
      run += c[k];
    }
    carry += tile;
    __syncthreads();
  }
  // Longest row: wave max, then across waves.
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off));
  if (lane == 0) wmax[wave] = mx;
  __syncthreads();
  if (tid == 0) {
    int m = 0;
    for (int w = 0; w < 16; ++w) m = max(m, wmax[w]);
    row_ptr[n] = static_cast<int32_t>(carry);
    totals[0] = carry;
    totals[1] = m;
    totals[2] = carry >= 0x7fffffffLL ? 1 : 0;
  }
}

// ---------------------------------------------------------------------------
// Block-sparse attention, bf16, 8x8 tiles.
//
// Work decomposition.  A workgroup of 4 * GR waves owns a group of GR x 2
// query tiles of one frame (GR = 2 or 3, chosen per plan) and walks the
// ascending union of their tile lists, prepared by the plan
// (group_list_kernel).  Each key tile is streamed once per workgroup into one
// of two LDS buffers by range-checked buffer DMA (buffer_load_dwordx4 ... lds),
// so the next tile streams in while the current one is consumed, and all
// waves use it: a 3 x 2 group loads each key tile once for 384 queries.  A
// wave owns 32 queries (lane % 32 = query) and skips a 32-key half of a tile
// whenever none of its queries retains a key there: tiles that only the other
// query tiles of the group need cost loads but no matrix work.
//
//   S^T (keys x queries) = K Q^T :  A = K rows from LDS, B = Q^T in registers
//   O^T (d x queries)   += V^T P^T : A = V^T via ds_read_b64_tr_b16, B = P^T
// The 32x32 output layout puts key rows {8(i/4) + 4(lane/32) + i%4} of a
// 32-key block in register i of a lane, which is exactly the k-slot order of
// the next MFMA's B operand, so P never leaves registers.
// ---------------------------------------------------------------------------
// LDS row strides (bytes) of the staged K and V tiles.  K rows are read as
// 16-byte MFMA operands by 16 lanes at a time (same chunk, 16 consecutive rows):
// a stride of 4 banks mod 64 spreads them over all banks.  V rows are read with
// ds_read_b64_tr_b16 by 32 lanes at a time (4 consecutive rows x 64 bytes): a
// stride of 16 banks mod 64 does the same.  Both make every LDS address a
// per-lane base plus an immediate offset.
template <int D> struct AttnLds {
  static constexpr int KSTR = 2 * D + 16;
  static constexpr int VSTR = 2 * D + 64;
  static constexpr int KSEG = 64 * KSTR / 1024;  // 1 KB DMA segments per K tile
  static constexpr int VSEG = 64 * VSTR / 1024;
  static constexpr int BUF = (KSEG + VSEG) * 1024;
  static_assert(64 * KSTR % 1024 == 0 && 64 * VSTR % 1024 == 0, "tile must be whole segments");
};

template <int D, int METRIC, bool BLOCK, int GR>
__global__ __launch_bounds__(256 * GR, 1) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, const int16_t* __restrict__ lv,
    const int32_t* __restrict__ r2c, const int32_t* __restrict__ r2off,
    const int32_t* __restrict__ dmax, int n_r2c, int row_base, Grid g, int ngh, int ngw, int n_groups,
    const int32_t* __restrict__ gptr, const int2* __restrict__ glist,
    const int32_t* __restrict__ glen, const uint8_t* __restrict__ perm, int self_ref) {
  using L = AttnLds<D>;
  constexpr int NTHREADS = 256 * GR;
  constexpr int NWAVES = NTHREADS / 64;
  constexpr int KS = D / 16;  // k-steps of S^T
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  constexpr int NONE = 0x7fffffff;
  __shared__ __attribute__((aligned(1024))) char kv0[L::BUF];  // K | V, buffer 0
  __shared__ __attribute__((aligned(1024))) char kv1[L::BUF];  // K | V, buffer 1
  extern __shared__ int32_t r2s[];  // compact radius table (dynamic LDS)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int h = lane >> 5, col = lane & 31;
  // Dispatch goes round-robin over the 8 XCDs; give each XCD a contiguous
  // range of groups so that neighbouring groups, which share most key tiles,
  // run under the same L2.  The grid is padded to a multiple of 8.
  const int per_xcd = gridDim.x / 8;
  const int gid = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (gid >= n_groups) return;  // uniform over the workgroup, before any barrier
  for (int i = threadIdx.x; i < n_r2c; i += NTHREADS) r2s[i] = r2c[i];
  __syncthreads();

  // Group = GR x 2 query tiles of one frame.
  const int groups_per_frame = ngh * ngw;
  const int per_head = g.T * groups_per_frame;
  const int bh = gid / per_head;
  const int grem = gid % per_head;
  const int tq = grem / groups_per_frame;
  const int gr = (grem % groups_per_frame) / ngw, gc = grem % ngw;
  const size_t N = static_cast<size_t>(g.T) * g.H * g.W;

  // This wave: tile row gr*GR + wave/4, tile column gc*2 + wcol, query rows
  // 4*(wave%2)..+3 of that tile; lane%32 -> query.  Waves w, w+4 (and w+8)
  // share a SIMD; they take tiles of different rows and alternating columns,
  // so that a key tile listed by one row or one column of the group keeps
  // every SIMD busy.
  const int wcol = ((wave >> 1) ^ (wave >> 2)) & 1;
  int hq, wq, mbit;
  bool qvalid;
  if (perm) {
    // Regrouped (2 x 2 groups only): the wave's queries are entries
    // 32*wave .. +31 of the group's level order, anywhere in the group's
    // 16 x 16 positions, so every tile the group lists may hold keys for them.
    const int slot = perm[static_cast<size_t>(gid) * GROUP_SLOTS + 32 * wave + col];
    hq = gr * 16 + (slot >> 4);
    wq = gc * 16 + (slot & 15);
    mbit = 0xf;
    qvalid = hq < g.H && wq < g.W;
  } else {
    const int tc = gc * 2 + wcol;
    const int trq = gr * GR + (wave >> 2);
    wq = tc * 8 + (col & 7);
    hq = trq * 8 + 4 * (wave & 1) + (col >> 3);
    // This wave's query tile in the group's membership bits (see group_list_kernel).
    mbit = 1 << (2 * (wave >> 2) + wcol);
    qvalid = tc < g.nw && trq < g.nh && hq < g.H && wq < g.W;
  }
  [[maybe_unused]] const int nqh = (tq * g.H + hq) * g.W + wq;  // raster index (1-D window mask)
  const size_t nq = (static_cast<size_t>(tq) * g.H + (qvalid ? hq : 0)) * g.W + (qvalid ? wq : 0);
  bf16x8 qf[KS];
  {
    const uint16_t* qp = q + (static_cast<size_t>(bh) * N + nq) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * h);
  }
  const int trow = qvalid ? lv[static_cast<size_t>(bh) * N + nq] - row_base : 0;
  const int toff = r2off[trow];
  const int tdmax = qvalid ? dmax[trow] : -1;

  // The union of the two query tiles' tile lists, ascending, prepared by the
  // plan: entry (frame | ragged << 31, row0 | col0 << 16).  It is read through
  // 64-entry windows held in VGPRs (lane i holds entry 64*w + i) and taken out
  // with v_readlane; the window after the current one is loaded when the
  // current one is entered, long before its first use.  (Vector loads keep the
  // list out of the LDS wait counter: a scalar load in flight would hold up
  // every LDS wait.)
  const int n_tiles = glen[gid];
  const int2* lst = glist + gptr[gid];
  int2 cur = lane < n_tiles ? lst[lane] : make_int2(0, 0);
  int2 nxt = 64 + lane < n_tiles ? lst[64 + lane] : make_int2(0, 0);
  struct TileGeo {
    int tk, kr0, kc0, member;
    bool ragged;
  };
  // Entry j (entries are read in order, each once).
  auto entry = [&](int j) {
    if ((j & 63) == 0 && j > 0) {
      cur = nxt;
      nxt = j + 64 + lane < n_tiles ? lst[j + 64 + lane] : make_int2(0, 0);
    }
    const int ex = __builtin_amdgcn_readlane(cur.x, j & 63);
    const int ey = __builtin_amdgcn_readlane(cur.y, j & 63);
    return TileGeo{ex & 0xffff, ey & 0xffff, ey >> 16, (ex >> 16) & 0x3f, ex < 0};
  };

  // One buffer resource per head for K and V: every tile, edge tiles
  // included, is loaded with the interior address pattern.  A key position
  // outside the grid then reads a neighbouring token of the same head (or
  // zero past the head's end); such keys are always masked.
  const i32x4 krsrc = make_rsrc(k + static_cast<size_t>(bh) * N * D, static_cast<uint32_t>(N * D * 2));
  const i32x4 vrsrc = make_rsrc(v + static_cast<size_t>(bh) * N * D, static_cast<uint32_t>(N * D * 2));

  // Streams key tile t into buffer buf.  DMA segment s (1 KB) receives lane
  // l's 16 bytes at s*1KB + 16*l; the lane fetches the (key row, chunk) that
  // the padded layout puts there (pad chunks re-fetch the row's first chunk).
  // Every wave issues the same number of DMA loads per tile (a wave without a
  // segment of its own repeats the last one, writing identical bytes), so the
  // loop's memory counters follow a fixed pattern.  A lane's byte offset from
  // the tile's first key is fixed per segment; it is computed once here, and a
  // load adds it to the tile's offset.
  constexpr int NK = (L::KSEG + NWAVES - 1) / NWAVES, NV = (L::VSEG + NWAVES - 1) / NWAVES;
  struct SegLane {
    int kr, kc, c;  // key row / column within the tile, 16-byte chunk
  };
  auto seg_lane = [&](int stride, int nseg, int i) {
    const int seg = min(wave + NWAVES * i, nseg - 1);
    const int ob = seg * 1024 + lane * 16;
    const int kk = ob / stride;
    const int c = (ob % stride) / 16;
    return SegLane{kk >> 3, kk & 7, c < D / 8 ? c : 0};
  };
  uint32_t koff[NK], voff[NV];
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const SegLane sl = seg_lane(L::KSTR, L::KSEG, i);
    koff[i] = static_cast<uint32_t>((sl.kr * g.W + sl.kc) * D * 2 + sl.c * 16);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const SegLane sl = seg_lane(L::VSTR, L::VSEG, i);
    voff[i] = static_cast<uint32_t>((sl.kr * g.W + sl.kc) * D * 2 + sl.c * 16);
  }
  auto lds_seg = [&](char* dst, int nseg, int i) {
    return __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(dst))) +
        min(wave + NWAVES * i, nseg - 1) * 1024);
  };
  auto issue = [&](const TileGeo& t, char* buf) {
    char* vbuf = buf + L::KSEG * 1024;
    const uint32_t tile_bytes = static_cast<uint32_t>((t.tk * g.H + t.kr0) * g.W + t.kc0) * (D * 2u);
#pragma unroll
    for (int i = 0; i < NK; ++i)
      if (NWAVES * (L::KSEG / NWAVES) == L::KSEG || wave + NWAVES * i < L::KSEG)
        lds_dma16_buf(krsrc, tile_bytes + koff[i], lds_seg(buf, L::KSEG, i));
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (NWAVES * (L::VSEG / NWAVES) == L::VSEG || wave + NWAVES * i < L::VSEG)
        lds_dma16_buf(vrsrc, tile_bytes + voff[i], lds_seg(vbuf, L::VSEG, i));
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = (f32x16){0.f};
  float lsum = 0.f;
  const float c1 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  // The softmax reference (log2 units).  When the plan lists every query's
  // own tile (self_ref), it starts at the query's score with its own key,
  // which every generator retains and the loop therefore visits: kept
  // probabilities cannot all underflow, and no block has to be formed twice
  // just to set a first reference.  Otherwise it starts at -inf and the first
  // block with a kept key sets it.  Each lane of a query pair holds half of
  // the dot product.
  float mref = TRA_NEG_INF;
  if (self_ref) {
    const uint16_t* kp = k + (static_cast<size_t>(bh) * N + nq) * D;
    float dot = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 kv = *reinterpret_cast<const uint4*>(kp + 16 * ks + 8 * h);
      const uint4 qv = __builtin_bit_cast(uint4, qf[ks]);
      dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qv.x), __builtin_bit_cast(bf16x2, kv.x), dot, false);
      dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qv.y), __builtin_bit_cast(bf16x2, kv.y), dot, false);
      dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qv.z), __builtin_bit_cast(bf16x2, kv.z), dot, false);
      dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qv.w), __builtin_bit_cast(bf16x2, kv.w), dot, false);
    }
    dot += __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(dot)));
    mref = dot * c1;
  }
  // Per-lane LDS byte bases; every read below adds a compile-time offset.
  const int g4 = lane >> 4, r4 = (lane & 15) >> 2, j4 = lane & 3;
  const int kread = col * L::KSTR + h * 16;
  const int vread = (4 * (g4 >> 1) + r4) * L::VSTR + (16 * (g4 & 1) + 4 * j4) * 2;
  const int partner = (lane ^ 32) << 2;  // ds_bpermute address of the other half

  // S^T block blk (keys 32*blk..+31 of the tile x this wave's 32 queries).
  // The K fragments are read in NP parts, each part's reads before its MFMAs
  // (the scheduling fence keeps the compiler from spreading the reads between
  // the MFMAs, where each pair of them would wait out a full LDS latency): one
  // part with two waves per SIMD, two with three, whose registers are fewer.
  auto scores = [&](const char* buf, int blk) {
    constexpr int NP = GR == 3 ? 2 : 1, KP = KS / NP;
    f32x16 acc = (f32x16){0.f};
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      bf16x8 af[KP];
#pragma unroll
      for (int ks = 0; ks < KP; ++ks)
        af[ks] = *reinterpret_cast<const bf16x8*>(buf + kread + 32 * blk * L::KSTR + 32 * (pp * KP + ks));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KP; ++ks)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], qf[pp * KP + ks], acc, 0, 0, 0);
    }
    return acc;
  };
  // Online softmax of one 32-key block.  msk[x] holds the radius mask of
  // elements 2x, 2x+1 as two 16-bit halves (all ones = keep); it is applied
  // to the packed bf16 probabilities, and the running sum adds the same bf16
  // values the PV product uses.
  //
  // Lazy rescale: the reference (shared by both lanes of a query) moves only
  // when the kept probabilities of a lane's block, formed against it, sum to
  // more than 2^10 (so between moves every kept probability is <= 2^10), or
  // while it is unset.  The probabilities and their sum are formed first; the
  // test on the sum (which the running sum needs anyway) then decides, rarely,
  // to move the reference to the exact masked maximum and form them again.
  // P^T as the two 16-key B operands of the PV product; returns the block's
  // contribution to the running sum.
  auto probs = [&](const f32x16& sacc, const uint32_t* msk, bf16x8* pf) {
    // With no reference yet (-inf) the block is formed against 0 and formed
    // again once the reference has moved; if it cannot move (no kept key in
    // the block), every probability is masked.
    const float msub = mref == TRA_NEG_INF ? 0.f : mref;
    const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
    float ls[2] = {0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t pk[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[8 * j + 2 * x], c1, -msub));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[8 * j + 2 * x + 1], c1, -msub));
        pk[x] = pack_bf16x2(p0, p1) & msk[4 * j + x];
        ls[j] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[x]), ones, ls[j], false);
      }
      pf[j] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
    }
    return ls[0] + ls[1];
  };
  // Moves the reference to the exact masked maximum of the block where that
  // exceeds it (rare path).
  auto move_ref = [&](const f32x16& sacc, const uint32_t* msk) {
    float mx = TRA_NEG_INF;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int keep = (i & 1) ? static_cast<int>(msk[i >> 1]) >> 16
                               : static_cast<int>(msk[i >> 1] << 16) >> 16;
      mx = fmaxf(mx, __int_as_float((__float_as_int(sacc[i]) & keep) |
                                    (__float_as_int(TRA_NEG_INF) & ~keep)));
    }
    mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_bpermute(partner, __float_as_int(mx))));
    if (__any(mx * c1 > mref)) {
      const float mn = fmaxf(mref, mx * c1);
      const float alpha = mref == TRA_NEG_INF ? 0.f : __builtin_amdgcn_exp2f(mref - mn);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      mref = mn;
    }
  };
  // softmax step of one block: returns P^T in pf and updates the running sum.
  auto softmax = [&](const f32x16& sacc, const uint32_t* msk, bf16x8* pf) {
    float ls = probs(sacc, msk, pf);
    if (__any(!(ls <= 1024.f) || mref == TRA_NEG_INF)) {
      move_ref(sacc, msk);
      ls = probs(sacc, msk, pf);
    }
    lsum += ls;
  };
  // O^T += V^T P^T for block blk.
  auto pv = [&](const char* buf, int blk, const bf16x8* pf) {
    const char* vb = buf + L::KSEG * 1024 + vread;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint2 lo = lds_read_tr_b(vb + (32 * blk + 16 * j) * L::VSTR + 64 * db);
        const uint2 hi = lds_read_tr_b(vb + (32 * blk + 16 * j + 8) * L::VSTR + 64 * db);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[j], oacc[db], 0, 0, 0);
      }
    }
  };

  // Radius mask.  Key (kr0 + 4*blk + a, kc0 + 4*h + b) sits in register
  // i = 4a + b of block blk; it is kept iff dw2[b] < rr[4*blk + a], with
  // dw2[b] = (w_q - w_k)^2 and rr = R2 + 1 - (h_q - h_k)^2 (R2 = -1 for an
  // inactive frame).  Keys outside the grid get sentinels that fail the test:
  // rr <= 2^30 (radius tables stay below 2^30), so the differences below
  // stay inside int32.
  constexpr int COL_OUT = 0x40000001, ROW_OUT = -1;
  constexpr int WIN_COL_OUT = 0x20000000, WIN_ROW_OUT = -0x20000000;
  // When `more`, the LDS DMA of the next tile (tn into nbuf) is issued once
  // the score MFMAs are in flight, so that the matrix unit works while the
  // DMA instructions wait to issue.
  auto compute = [&](const TileGeo& t, const char* buf, bool more, const TileGeo& tn, char* nbuf) {
    int dw2[4], rr[8];
    [[maybe_unused]] int dn[8];
    bool doq[2] = {false, false};
    // The geometry is needed only by a wave whose query tile lists the key
    // tile (wave-uniform membership bit); the others only take part in the
    // next tile's loads.
    if (t.member & mbit) {
      const int delta = t.tk > tq ? t.tk - tq : tq - t.tk;
      const int tv = r2s[toff + min(delta, max(tdmax, 0))];
      const int thr1 = delta <= tdmax ? tv + 1 : 0;
      const int dwa = wq - t.kc0 - 4 * h;
      const int dha = hq - t.kr0;
      if constexpr (BLOCK) {  // block-only mask: every key of a listed tile inside the grid
#pragma unroll
        for (int b = 0; b < 4; ++b) dw2[b] = 0;
#pragma unroll
        for (int a = 0; a < 8; ++a) rr[a] = 1;
      } else if constexpr (METRIC == METRIC_WINDOW) {
        // 1-D window: key (a, b) is kept iff |x| <= rho, x = base - a*W - b the
        // query's raster index minus the key's.  Upper bound: -b < rr[a]; lower
        // bound: b < dn[a].
        const int rho = delta <= tdmax ? tv : -1;
        const int base = nqh - ((t.tk * g.H + t.kr0) * g.W + t.kc0 + 4 * h);
#pragma unroll
        for (int b = 0; b < 4; ++b) dw2[b] = -b;
#pragma unroll
        for (int a = 0; a < 8; ++a) {
          rr[a] = rho - base + a * g.W + 1;
          dn[a] = rho + base - a * g.W + 1;
        }
      } else if constexpr (METRIC == METRIC_L1) {
#pragma unroll
        for (int b = 0; b < 4; ++b) dw2[b] = abs(dwa - b);
#pragma unroll
        for (int a = 0; a < 8; ++a) rr[a] = thr1 - abs(dha - a);
      } else {
        dw2[0] = __mul24(dwa, dwa);
#pragma unroll
        for (int b = 1; b < 4; ++b) dw2[b] = dw2[b - 1] - 2 * dwa + (2 * b - 1);
        rr[0] = thr1 - __mul24(dha, dha);
#pragma unroll
        for (int a = 1; a < 8; ++a) rr[a] = rr[a - 1] + 2 * dha - (2 * a - 1);
      }
      if (t.ragged) {  // tile at the bottom/right edge of the grid (wave-uniform)
        // The window's entries span up to 2^26 either side of zero, so its
        // sentinels are +-2^29: their differences (up to 2^30) stay inside int32
        // also where an out-of-grid row meets an out-of-grid column.
#pragma unroll
        for (int b = 0; b < 4; ++b)
          if (t.kc0 + 4 * h + b >= g.W) dw2[b] = METRIC == METRIC_WINDOW ? WIN_COL_OUT : COL_OUT;
#pragma unroll
        for (int a = 0; a < 8; ++a)
          if (t.kr0 + a >= g.H) rr[a] = METRIC == METRIC_WINDOW ? WIN_ROW_OUT : ROW_OUT;
      }
      const int mindw = min(min(dw2[0], dw2[1]), min(dw2[2], dw2[3]));
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int* r = rr + 4 * blk;
        if constexpr (METRIC == METRIC_WINDOW && !BLOCK) {
          // Some b in [0, 3] with -b < rr[a] and b < dn[a] (edge columns count;
          // their masks drop them).
          bool any = false;
#pragma unroll
          for (int a = 4 * blk; a < 4 * blk + 4; ++a) any |= max(0, 1 - rr[a]) <= min(3, dn[a] - 1);
          doq[blk] = __any(any);
        } else {
          doq[blk] = __any(mindw < max(max(r[0], r[1]), max(r[2], r[3])));
        }
      }
    }
    // Sign bytes of the two differences -> 16-bit keep masks of block blk.
    auto masks = [&](int blk, uint32_t* msk) {
      if (BLOCK && !t.ragged) {
#pragma unroll
        for (int x = 0; x < 8; ++x) msk[x] = 0xffffffffu;
        return;
      }
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int ra = rr[4 * blk + (x >> 1)];
        int t0 = dw2[2 * (x & 1)] - ra, t1 = dw2[2 * (x & 1) + 1] - ra;
        if constexpr (METRIC == METRIC_WINDOW && !BLOCK) {
          const int da = dn[4 * blk + (x >> 1)];
          t0 &= 2 * (x & 1) - da;
          t1 &= 2 * (x & 1) + 1 - da;
        }
        msk[x] = __builtin_amdgcn_perm(static_cast<uint32_t>(t1), static_cast<uint32_t>(t0), 0x0B0B0909u);
      }
    };
    // The two blocks run one after the other (one code path per block, no
    // separate path for "both"): with a single path the compiler keeps the
    // output accumulators in place across the loop instead of copying them
    // between register sets, which costs more than the lost overlap.
    bool issued = !more;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      if (doq[blk]) {
        uint32_t m[8];
        const f32x16 sacc = scores(buf, blk);
        masks(blk, m);
        if (!issued) issue(tn, nbuf);
        issued = true;
        bf16x8 pf[2];
        softmax(sacc, m, pf);
        pv(buf, blk, pf);
      }
    }
    if (!issued) issue(tn, nbuf);
  };

  // One barrier per key tile.  At the barrier of tile e every wave has its
  // own DMA loads of tile e complete (the only ones outstanding) and has
  // finished computing tile e-1, so the data of e is visible and the other
  // buffer is free: tile e+1 is then streamed into it while e is consumed.
  if (n_tiles > 0) {
    TileGeo tc = entry(0), tn;
    issue(tc, kv0);
    int e = 0;
    while (true) {
      wait_vmcnt<0>();
      lds_barrier();
      const bool more0 = e + 1 < n_tiles;
      if (more0) tn = entry(e + 1);
      compute(tc, kv0, more0, tn, kv1);
      if (++e == n_tiles) break;
      tc = tn;
      wait_vmcnt<0>();
      lds_barrier();
      const bool more1 = e + 1 < n_tiles;
      if (more1) tn = entry(e + 1);
      compute(tc, kv1, more1, tn, kv0);
      if (++e == n_tiles) break;
      tc = tn;
    }
  }

  const float ltot = lsum + __int_as_float(__builtin_amdgcn_ds_bpermute(partner, __float_as_int(lsum)));
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (qvalid) {
    uint16_t* op = o + (static_cast<size_t>(bh) * N + nq) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = 32 * db + 8 * a + 4 * h;
        const uint2 out4 = make_uint2(pack_bf16x2(oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv),
                                      pack_bf16x2(oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv));
        *reinterpret_cast<uint2*>(op + d0) = out4;
      }
  }
}

// fp32 inputs: a workgroup of f32_split<D> waves per query tile, lane =
// query (tile-local row-major).  The work units are the half key tiles (32
// keys: rows 0-3 or 4-7) of the tile's list; wave w takes units w, w + S, ...
// into its own LDS slot and runs an fp32 online softmax over them.  The
// waves' partial states (reference, sum, accumulator) are then merged in
// pairs through LDS.  The split puts S waves to work per query tile on small
// grids, two per SIMD at d = 64.
template <int D> constexpr int f32_split() { return D == 64 ? 8 : 4; }  // 128 KB of LDS either way
template <int D, int METRIC, bool BLOCK>
__global__ __launch_bounds__(64 * f32_split<D>()) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, const int16_t* __restrict__ lv, const int32_t* __restrict__ r2,
    int row_base, int T, Grid g, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx) {
  constexpr int S = f32_split<D>();
  __shared__ float kv_lds[S][2][32][D];  // per wave: K rows, V rows of its current half tile
  static_assert((S / 2) * 64 * (D + 2) <= S * 2 * 32 * D, "a merge round fits in the tile slots");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x;
  const int bh = row / g.count, tile = row % g.count;
  const size_t N = static_cast<size_t>(g.T) * g.H * g.W;
  const int tq = tile / g.per_frame, trem = tile % g.per_frame;
  const int h0 = (trem / g.nw) * 8, w0 = (trem % g.nw) * 8;
  const int hq = h0 + (lane >> 3), wq = w0 + (lane & 7);
  const bool qvalid = hq < g.H && wq < g.W;
  const size_t nq = (static_cast<size_t>(tq) * g.H + (qvalid ? hq : h0)) * g.W + (qvalid ? wq : w0);
  float qr[D], acc[D];
  const float* qp = q + (static_cast<size_t>(bh) * N + nq) * D;
#pragma unroll
  for (int dd = 0; dd < D; ++dd) {
    qr[dd] = qp[dd];
    acc[dd] = 0.f;
  }
  const int trow = qvalid ? lv[static_cast<size_t>(bh) * N + nq] - row_base : 0;
  const int32_t* r2row = r2 + trow * T;
  const float scale = 1.f / sqrtf(static_cast<float>(D));
  float mref = TRA_NEG_INF, lsum = 0.f;
  const float* kbase = k + static_cast<size_t>(bh) * N * D;
  const float* vbase = v + static_cast<size_t>(bh) * N * D;
  float (*k_lds)[D] = kv_lds[wave][0];
  float (*v_lds)[D] = kv_lds[wave][1];
  const int beg = row_ptr[row], end = row_ptr[row + 1];
  const int units = 2 * (end - beg);
  const int steps = (units + S - 1) / S;  // the same for every wave of the workgroup
  for (int it = 0; it < steps; ++it) {
    const int u = it * S + wave;
    const bool have = u < units;  // wave-uniform
    const int kt = have ? col_idx[beg + (u >> 1)] : 0;
    const int tk = kt / g.per_frame, krem = kt % g.per_frame;
    const int kr0 = (krem / g.nw) * 8 + 4 * (u & 1), kc0 = (krem % g.nw) * 8;
    __syncthreads();
    if (have) {
      for (int idx = lane; idx < 32 * D / 4; idx += 64) {
        const int kk = idx / (D / 4), c = idx % (D / 4);
        const int kr = min(kr0 + (kk >> 3), g.H - 1), kc = min(kc0 + (kk & 7), g.W - 1);
        const size_t nk = (static_cast<size_t>(tk) * g.H + kr) * g.W + kc;
        *reinterpret_cast<float4*>(&k_lds[kk][4 * c]) = *reinterpret_cast<const float4*>(kbase + nk * D + 4 * c);
        *reinterpret_cast<float4*>(&v_lds[kk][4 * c]) = *reinterpret_cast<const float4*>(vbase + nk * D + 4 * c);
      }
    }
    __syncthreads();
    if (have) {
      const int delta = tk > tq ? tk - tq : tq - tk;
      const int thr = qvalid ? r2row[delta] : -1;
      for (int kk = 0; kk < 32; ++kk) {
        const int kr = kr0 + (kk >> 3), kc = kc0 + (kk & 7);
        const int dh = hq - kr, dw = wq - kc;
        if (kr >= g.H || kc >= g.W) continue;
        if (!BLOCK) {
          if (thr < 0) continue;
          if (METRIC == METRIC_WINDOW) {
            const long long dn = static_cast<long long>(nq) - ((static_cast<long long>(tk) * g.H + kr) * g.W + kc);
            if (dn > thr || -dn > thr) continue;
          } else if ((METRIC == METRIC_L1 ? abs(dh) + abs(dw) : dh * dh + dw * dw) > thr) {
            continue;
          }
        }
        float sc = 0.f;
#pragma unroll
        for (int dd = 0; dd < D; ++dd) sc = fmaf(qr[dd], k_lds[kk][dd], sc);
        sc *= scale;
        if (sc > mref) {
          const float alpha = expf(mref - sc);
          lsum *= alpha;
#pragma unroll
          for (int dd = 0; dd < D; ++dd) acc[dd] *= alpha;
          mref = sc;
        }
        const float p = expf(sc - mref);
        lsum += p;
#pragma unroll
        for (int dd = 0; dd < D; ++dd) acc[dd] = fmaf(p, v_lds[kk][dd], acc[dd]);
      }
    }
  }
  // Pairwise merge: in each round the upper half of the remaining waves
  // writes its state, and wave w of the lower half folds in wave w + half's.
  // A state without a kept key (reference -inf) adds nothing.
  float* st = &kv_lds[0][0][0][0];
#pragma unroll
  for (int half = S / 2; half >= 1; half /= 2) {
    __syncthreads();
    if (wave >= half && wave < 2 * half) {
      float* mine = st + ((wave - half) * 64 + lane) * (D + 2);
      mine[0] = mref;
      mine[1] = lsum;
#pragma unroll
      for (int dd = 0; dd < D; ++dd) mine[2 + dd] = acc[dd];
    }
    __syncthreads();
    if (wave < half) {
      const float* other = st + (wave * 64 + lane) * (D + 2);
      const float mo = other[0];
      const float M = fmaxf(mref, mo);
      const float fa = mref == TRA_NEG_INF ? 0.f : expf(mref - M);
      const float fb = mo == TRA_NEG_INF ? 0.f : expf(mo - M);
      lsum = lsum * fa + other[1] * fb;
#pragma unroll
      for (int dd = 0; dd < D; ++dd) acc[dd] = acc[dd] * fa + other[2 + dd] * fb;
      mref = M;
    }
  }
  if (wave == 0 && qvalid) {
    float* op = o + (static_cast<size_t>(bh) * N + nq) * D;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;  // no key under a vote threshold: O = 0
#pragma unroll
    for (int dd = 0; dd < D; ++dd) op[dd] = acc[dd] * inv;
  }
}

// ---------------------------------------------------------------------------
// Exact pair counts.
// ---------------------------------------------------------------------------
template <int METRIC>
__global__ __launch_bounds__(256) void retained_kernel(const int16_t* __restrict__ lv,
                                                      const int32_t* __restrict__ r2, int T,
                                                      int row_base, Grid g, int64_t n_total,
                                                      unsigned long long* __restrict__ out) {
  __shared__ unsigned long long part[256];
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  unsigned long long cnt = 0;
  if (i < n_total) {
    const int64_t N = static_cast<int64_t>(g.T) * g.H * g.W;
    const int64_t n = i % N;
    const int t = static_cast<int>(n / (g.H * g.W)), hh = static_cast<int>((n / g.W) % g.H),
              ww = static_cast<int>(n % g.W);
    const int32_t* row = r2 + (lv[i] - row_base) * T;
    if (METRIC == METRIC_WINDOW) {
      const int64_t rho = row[0];
      cnt = static_cast<unsigned long long>(min(N - 1, n + rho) - max(int64_t(0), n - rho) + 1);
    } else {
      constexpr bool L1 = METRIC == METRIC_L1;
      for (int tk = 0; tk < T; ++tk) {
        const int thr = row[tk > t ? tk - t : t - tk];
        if (thr < 0) continue;
        const int rad = mask_reach<L1>(thr);
        for (int hk = max(0, hh - rad); hk <= min(g.H - 1, hh + rad); ++hk) {
          const int a = mask_half_width<L1>(thr, hk - hh);
          cnt += min(g.W - 1, ww + a) - max(0, ww - a) + 1;
        }
      }
    }
  }
  part[threadIdx.x] = cnt;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) part[threadIdx.x] += part[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicAdd(out, part[0]);
}

__global__ __launch_bounds__(256) void listed_kernel(Grid g, int64_t n_rows,
                                                    const int32_t* __restrict__ row_ptr,
                                                    const int32_t* __restrict__ col_idx,
                                                    unsigned long long* __restrict__ out) {
  __shared__ unsigned long long part[256];
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  unsigned long long cnt = 0;
  if (r < n_rows) {
    auto valid = [&](int t) {
      const int rem = t % g.per_frame;
      const int h0 = (rem / g.nw) * g.th, w0 = (rem % g.nw) * g.tw;
      return static_cast<unsigned long long>(min(g.th, g.H - h0) * min(g.tw, g.W - w0));
    };
    const unsigned long long nqv = valid(static_cast<int>(r % g.count));
    for (int e = row_ptr[r]; e < row_ptr[r + 1]; ++e) cnt += nqv * valid(col_idx[e]);
  }
  part[threadIdx.x] = cnt;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) part[threadIdx.x] += part[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicAdd(out, part[0]);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_pool(int dtype, int d, const void* k, void* kbar, int BH, const Grid& pool,
                       hipStream_t s) {
  const dim3 grid(pool.count, BH), block(256);
  if (dtype == 1) {
    if (d == 128) pool_kernel<128, true><<<grid, block, 0, s>>>(k, kbar, pool);
    else pool_kernel<64, true><<<grid, block, 0, s>>>(k, kbar, pool);
  } else {
    if (d == 128) pool_kernel<128, false><<<grid, block, 0, s>>>(k, kbar, pool);
    else pool_kernel<64, false><<<grid, block, 0, s>>>(k, kbar, pool);
  }
  return hipGetLastError();
}

hipError_t launch_entropy(int dtype, int d, const void* q, const void* kbar, const float* pool_w,
                          int BH, int N, const Grid& pool, const EntropyArgs& ea, float* H_out,
                          int16_t* lv_out, hipStream_t s) {
  const dim3 grid((N + 255) / 256, BH), block(256);
  const int n_pool = pool.count;
  if (dtype == 1) {
    const auto* qq = static_cast<const uint16_t*>(q);
    const auto* kb = static_cast<const uint16_t*>(kbar);
    const dim3 grid16((N + ENT_QPW - 1) / ENT_QPW, BH), block16(ENT_WAVES * 64);
    const int nfull = pool_full_count(pool);
    const float wfull = static_cast<float>(pool.th * pool.tw);
    if (d == 128)
      entropy_bf16_kernel<128><<<grid16, block16, 0, s>>>(qq, kb, pool_w, N, n_pool, nfull, wfull, ea, H_out, lv_out);
    else
      entropy_bf16_kernel<64><<<grid16, block16, 0, s>>>(qq, kb, pool_w, N, n_pool, nfull, wfull, ea, H_out, lv_out);
  } else {
    const auto* qq = static_cast<const float*>(q);
    const auto* kb = static_cast<const float*>(kbar);
    if (d == 128) entropy_f32_kernel<128><<<grid, block, 0, s>>>(qq, kb, pool_w, N, n_pool, ea, H_out, lv_out);
    else entropy_f32_kernel<64><<<grid, block, 0, s>>>(qq, kb, pool_w, N, n_pool, ea, H_out, lv_out);
  }
  return hipGetLastError();
}

hipError_t launch_fill_levels(int16_t* lv, float* H, int64_t n, hipStream_t s) {
  fill_levels_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(lv, H, n);
  return hipGetLastError();
}

static int log2i(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

hipError_t launch_csr_runs(bool l1, const int16_t* lv, const RadiusTable& tab, int n_levels, int row_base,
                           int BH, const Grid& tiles, int DM, int32_t* counts, int32_t* runs, int32_t* rowwin,
                           hipStream_t s, int group_rows, const int32_t* gptr, int32_t* glist, int32_t* glen) {
  const size_t lds = (2 * static_cast<size_t>(n_levels) + tab.n_r2c) * sizeof(int32_t);
  if (lds > 65536) return hipErrorInvalidValue;  // the parameter check bounds the table well below this
  if (glist && group_rows != 2 && group_rows != 3) return hipErrorInvalidValue;
  const int ngh = group_grid_rows(tiles, glist ? group_rows : 2), ngw = group_grid_cols(tiles);
  int2* gl = reinterpret_cast<int2*>(glist);
#define TRA_RUNS(L, G, GRID, NT)                                                                                  \
  csr_runs_kernel<L, G><<<GRID, NT, lds, s>>>(lv, tab.r2c, tab.r2off, tab.dmax, n_levels, tab.n_r2c, tab.T, row_base, \
                                             tiles, log2i(tiles.tw), DM, counts, runs, rowwin, ngh, ngw, gptr, gl, glen)
  if (glist && group_rows == 2) {
    const dim3 grid(tiles.T * ngh * ngw, BH);
    if (l1) TRA_RUNS(true, 2, grid, 256);
    else TRA_RUNS(false, 2, grid, 256);
  } else {
    // 3 x 2 groups merge their lists in a pass of their own: in this kernel
    // one wave would merge six tiles' runs while the other five wait (168
    // against 118 + 30 us at Wan2.1-14B 720p).
    const dim3 grid((tiles.count + 3) / 4, BH);
    if (l1) TRA_RUNS(true, 0, grid, 256);
    else TRA_RUNS(false, 0, grid, 256);
    if (glist) {
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_group_lists(true, BH, tiles, group_rows, DM, runs, rowwin, nullptr, nullptr, gptr, glist, glen, s);
    }
  }
#undef TRA_RUNS
  return hipGetLastError();
}

hipError_t launch_scan(const int32_t* counts, int64_t n_rows, int32_t* row_ptr, int64_t* totals,
                       hipStream_t s) {
  scan_kernel<<<1, 1024, 0, s>>>(counts, n_rows, row_ptr, totals);
  return hipGetLastError();
}

hipError_t launch_csr_expand(int BH, const Grid& tiles, int DM, const int32_t* runs,
                             const int32_t* rowwin, const int32_t* row_ptr, int32_t* col_idx,
                             hipStream_t s) {
  const int64_t n_rows = static_cast<int64_t>(BH) * tiles.count;
  csr_expand_kernel<<<static_cast<unsigned>((n_rows + 3) / 4), 256, 0, s>>>(tiles, DM, n_rows, runs, rowwin,
                                                                           row_ptr, col_idx);
  return hipGetLastError();
}

size_t attention_lds_bytes(int d, int n_r2c) {
  const size_t kv = d == 128 ? 2 * AttnLds<128>::BUF : 2 * AttnLds<64>::BUF;
  return kv + static_cast<size_t>(n_r2c) * sizeof(int32_t);
}

hipError_t launch_group_lists(bool fill, int BH, const Grid& tiles, int group_rows, int DM, const int32_t* runs,
                              const int32_t* rowwin, const int32_t* frow_ptr, const int32_t* fcol,
                              const int32_t* gptr, int32_t* glist, int32_t* glen, hipStream_t s) {
  if (group_rows != 2 && group_rows != 3) return hipErrorInvalidValue;
  const int ngh = group_grid_rows(tiles, group_rows), ngw = group_grid_cols(tiles);
  const int64_t n_groups = group_count(BH, tiles, group_rows);
  const unsigned grid = static_cast<unsigned>((n_groups + 3) / 4);
  auto* gl = reinterpret_cast<int2*>(glist);
#define TRA_GL(F, G) \
  group_list_kernel<F, G><<<grid, 256, 0, s>>>(tiles, DM, ngh, ngw, n_groups, runs, rowwin, frow_ptr, fcol, gptr, gl, glen)
  if (group_rows == 3) {
    if (fill) TRA_GL(true, 3);
    else TRA_GL(false, 3);
  } else {
    if (fill) TRA_GL(true, 2);
    else TRA_GL(false, 2);
  }
#undef TRA_GL
  return hipGetLastError();
}

hipError_t launch_window_csr(bool fill, const int16_t* lv, const int32_t* r2, const int32_t* dmax, int T,
                             int row_base, int BH, const Grid& tiles, const int32_t* row_ptr, int32_t* counts,
                             int32_t* col_idx, hipStream_t s) {
  const int64_t n_rows = static_cast<int64_t>(BH) * tiles.count;
  const unsigned grid = static_cast<unsigned>((n_rows + 3) / 4);
  if (fill)
    window_csr_kernel<true><<<grid, 256, 0, s>>>(lv, r2, dmax, T, row_base, tiles, n_rows, row_ptr, counts, col_idx);
  else
    window_csr_kernel<false><<<grid, 256, 0, s>>>(lv, r2, dmax, T, row_base, tiles, n_rows, row_ptr, counts, col_idx);
  return hipGetLastError();
}

hipError_t launch_window_groups(bool fill, const int16_t* lv, const int32_t* r2, const int32_t* dmax, int T,
                                int row_base, int BH, const Grid& tiles, int group_rows, const int32_t* gptr,
                                int32_t* glist, int32_t* glen, hipStream_t s) {
  if (group_rows != 2 && group_rows != 3) return hipErrorInvalidValue;
  const int ngh = group_grid_rows(tiles, group_rows), ngw = group_grid_cols(tiles);
  const int64_t n_groups = group_count(BH, tiles, group_rows);
  const unsigned grid = static_cast<unsigned>((n_groups + 3) / 4);
  auto* gl = reinterpret_cast<int2*>(glist);
#define TRA_WG(F, G) \
  window_group_kernel<F, G><<<grid, 256, 0, s>>>(lv, r2, dmax, T, row_base, tiles, ngh, ngw, n_groups, gptr, gl, glen)
  if (group_rows == 3) {
    if (fill) TRA_WG(true, 3);
    else TRA_WG(false, 3);
  } else {
    if (fill) TRA_WG(true, 2);
    else TRA_WG(false, 2);
  }
#undef TRA_WG
  return hipGetLastError();
}

hipError_t launch_votes(bool l1, const int16_t* lv, const int32_t* r2, const int32_t* dmax, int T, int row_base,
                        int BH, const Grid& tiles, const int32_t* row_ptr, const int32_t* col_idx, int theta,
                        int16_t* votes, int32_t* counts2, unsigned long long* kept_votes, hipStream_t s) {
  const int64_t n_rows = static_cast<int64_t>(BH) * tiles.count;
  const unsigned grid = static_cast<unsigned>((n_rows + 3) / 4);
  if (l1)
    vote_kernel<true><<<grid, 256, 0, s>>>(lv, r2, dmax, T, row_base, tiles, n_rows, row_ptr, col_idx, theta,
                                           votes, counts2, kept_votes);
  else
    vote_kernel<false><<<grid, 256, 0, s>>>(lv, r2, dmax, T, row_base, tiles, n_rows, row_ptr, col_idx, theta,
                                            votes, counts2, kept_votes);
  return hipGetLastError();
}

hipError_t launch_vote_compact(int64_t n_rows, const int32_t* row_ptr, const int32_t* col_idx, const int16_t* votes,
                               int theta, const int32_t* row_ptr2, int32_t* col_idx2, hipStream_t s) {
  vote_compact_kernel<<<static_cast<unsigned>((n_rows + 3) / 4), 256, 0, s>>>(n_rows, row_ptr, col_idx, votes, theta,
                                                                            row_ptr2, col_idx2);
  return hipGetLastError();
}

hipError_t launch_regroup(const int16_t* lv, int BH, const Grid& tiles, uint8_t* perm, hipStream_t s) {
  static_assert(GROUP_SLOTS == 32 * 8, "one slot per query lane of a 2 x 2 group's attention workgroup");
  const int ngh = group_grid_rows(tiles, 2), ngw = group_grid_cols(tiles);
  const int64_t groups = group_count(BH, tiles, 2);
  regroup_kernel<<<static_cast<unsigned>(groups), GROUP_SLOTS, 0, s>>>(lv, tiles, ngh, ngw, perm);
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, int d, const void* q, const void* k, const void* v,
                            void* o, const int16_t* lv, const RadiusTable& tab, int row_base,
                            int BH, const Grid& tiles, const int32_t* row_ptr,
                            const int32_t* col_idx, const int32_t* gptr, const int32_t* glist,
                            const int32_t* glen, int group_rows, const uint8_t* perm, bool block_mask,
                            bool self_ref, hipStream_t s) {
  const int32_t* r2 = tab.r2;
  const unsigned rows = static_cast<unsigned>(BH) * tiles.count;
  if (dtype == 1) {
    const auto* qq = static_cast<const uint16_t*>(q);
    const auto* kk = static_cast<const uint16_t*>(k);
    const auto* vv = static_cast<const uint16_t*>(v);
    auto* oo = static_cast<uint16_t*>(o);
    if (group_rows != 2 && group_rows != 3) return hipErrorInvalidValue;
    if (perm && group_rows != 2) return hipErrorInvalidValue;  // regrouping covers 2 x 2 groups
    const int ngh = group_grid_rows(tiles, group_rows), ngw = group_grid_cols(tiles);
    const int64_t groups = group_count(BH, tiles, group_rows);
    const unsigned grid = static_cast<unsigned>((groups + 7) / 8 * 8);
    const int ng = static_cast<int>(groups);
    const size_t lds_tab = static_cast<size_t>(tab.n_r2c) * sizeof(int32_t);
#define TRA_ATTN(DD, M, B, G)                                                                                   \
  attn_bf16_kernel<DD, M, B, G><<<grid, 256 * G, lds_tab, s>>>(qq, kk, vv, oo, lv, tab.r2c, tab.r2off, tab.dmax, \
                                                               tab.n_r2c, row_base, tiles, ngh, ngw, ng, gptr,     \
                                                               reinterpret_cast<const int2*>(glist), glen, perm,   \
                                                               self_ref ? 1 : 0)
#define TRA_ATTN_G(G)                                                  \
  do {                                                                 \
    if (block_mask) {                                                  \
      if (d == 128) TRA_ATTN(128, METRIC_L2, true, G);                 \
      else TRA_ATTN(64, METRIC_L2, true, G);                           \
    } else if (tab.metric == METRIC_L1) {                              \
      if (d == 128) TRA_ATTN(128, METRIC_L1, false, G);                \
      else TRA_ATTN(64, METRIC_L1, false, G);                          \
    } else if (tab.metric == METRIC_WINDOW) {                          \
      if (d == 128) TRA_ATTN(128, METRIC_WINDOW, false, G);            \
      else TRA_ATTN(64, METRIC_WINDOW, false, G);                      \
    } else {                                                           \
      if (d == 128) TRA_ATTN(128, METRIC_L2, false, G);                \
      else TRA_ATTN(64, METRIC_L2, false, G);                          \
    }                                                                  \
  } while (0)
    if (group_rows == 3) TRA_ATTN_G(3);
    else TRA_ATTN_G(2);
#undef TRA_ATTN_G
#undef TRA_ATTN
  } else {
    const auto* qq = static_cast<const float*>(q);
    const auto* kk = static_cast<const float*>(k);
    const auto* vv = static_cast<const float*>(v);
    auto* oo = static_cast<float*>(o);
#define TRA_ATTN32(DD, M, B) \
  attn_f32_kernel<DD, M, B><<<rows, 64 * f32_split<DD>(), 0, s>>>(qq, kk, vv, oo, lv, r2, row_base, tiles.T, tiles, \
                                                                 row_ptr, col_idx)
    if (block_mask) {
      if (d == 128) TRA_ATTN32(128, METRIC_L2, true);
      else TRA_ATTN32(64, METRIC_L2, true);
    } else if (tab.metric == METRIC_L1) {
      if (d == 128) TRA_ATTN32(128, METRIC_L1, false);
      else TRA_ATTN32(64, METRIC_L1, false);
    } else if (tab.metric == METRIC_WINDOW) {
      if (d == 128) TRA_ATTN32(128, METRIC_WINDOW, false);
      else TRA_ATTN32(64, METRIC_WINDOW, false);
    } else {
      if (d == 128) TRA_ATTN32(128, METRIC_L2, false);
      else TRA_ATTN32(64, METRIC_L2, false);
    }
#undef TRA_ATTN32
  }
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void level_diff_kernel(const int16_t* __restrict__ a,
                                                        const int16_t* __restrict__ b, int64_t n,
                                                        unsigned long long* __restrict__ out) {
  unsigned long long cnt = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    cnt += a[i] != b[i];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
  if ((threadIdx.x & 63) == 0 && cnt) atomicAdd(out, cnt);
}

__global__ __launch_bounds__(64) void clear_u64_kernel(unsigned long long* __restrict__ p, int n) {
  if (static_cast<int>(threadIdx.x) < n) p[threadIdx.x] = 0;
}
hipError_t launch_clear_counters(unsigned long long* p, int n, hipStream_t s) {
  if (n < 1 || n > 64) return hipErrorInvalidValue;
  clear_u64_kernel<<<1, 64, 0, s>>>(p, n);
  return hipGetLastError();
}
hipError_t launch_level_diff(const int16_t* a, const int16_t* b, int64_t n, unsigned long long* out,
                             hipStream_t s) {
  const int64_t blocks = (n + 255) / 256;
  level_diff_kernel<<<static_cast<unsigned>(blocks < 4096 ? blocks : 4096), 256, 0, s>>>(a, b, n, out);
  return hipGetLastError();
}

hipError_t launch_stats(int metric, const int16_t* lv, const int32_t* r2, int T, int row_base, int BH,
                        const Grid& tiles, const int32_t* row_ptr, const int32_t* col_idx,
                        unsigned long long* out2, hipStream_t s) {
  const int64_t nq = static_cast<int64_t>(BH) * tiles.T * tiles.H * tiles.W;
  const unsigned nb = static_cast<unsigned>((nq + 255) / 256);
  if (metric == METRIC_L1)
    retained_kernel<METRIC_L1><<<nb, 256, 0, s>>>(lv, r2, T, row_base, tiles, nq, out2);
  else if (metric == METRIC_WINDOW)
    retained_kernel<METRIC_WINDOW><<<nb, 256, 0, s>>>(lv, r2, T, row_base, tiles, nq, out2);
  else
    retained_kernel<METRIC_L2><<<nb, 256, 0, s>>>(lv, r2, T, row_base, tiles, nq, out2);
  const int64_t nr = static_cast<int64_t>(BH) * tiles.count;
  listed_kernel<<<static_cast<unsigned>((nr + 255) / 256), 256, 0, s>>>(tiles, nr, row_ptr, col_idx, out2 + 1);
  return hipGetLastError();
}

}  // namespace tra
