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
//   csr_kernel<FILL>      per query tile: union over its 64 queries of the disk
//                         footprints, as key-tile runs (count pass, fill pass)
//   scan_kernel           exclusive scan of the per-tile counts
//   attn_bf16_kernel      block-sparse flash attention: S^T = K Q^T and
//                         O^T += V^T P^T on 32x32x16 bf16 MFMA, K/V tiles staged
//                         in LDS (V read back transposed with ds_read_b64_tr_b16),
//                         exact radius mask in registers, fp32 online softmax
//   attn_f32_kernel       plain fp32 vector variant for fp32 inputs
//   stats kernels         exact retained / listed pair counts
#include "tra_internal.h"

#include <math.h>

namespace tra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

#define TRA_NEG_INF (-__builtin_inff())

__device__ __forceinline__ float bf16_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Integer square root floor(sqrt(x)) for 0 <= x < 2^31.
__device__ __forceinline__ int isqrt_i(int x) {
  long long r = static_cast<long long>(sqrtf(static_cast<float>(x)));
  r -= (r * r > x);
  r += ((r + 1) * (r + 1) <= x);
  return static_cast<int>(r);
}

// XOR swizzle of 16-byte chunks in an LDS tile whose rows are NCH chunks wide.
// Rows 0..15 map chunk c to distinct banks for both the 16-byte MFMA operand
// reads (16 rows, same chunk) and the transposing 8-byte reads (4 consecutive
// rows, 2 adjacent chunks).
template <int NCH>
__device__ __forceinline__ int swz(int r) {
  if constexpr (NCH == 16) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else {
    return ((r & 3) << 1) | ((r >> 2) & 1);
  }
}

// Transposing LDS read of 4 bf16 (ds_read_b64_tr_b16); elem_off in elements.
__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t* base, int elem_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)((__attribute__((address_space(3))) char*)(base) + elem_off * 2));
}

// Wave-wide min / max (64 lanes): DPP inside rows of 16, then lane swaps.
__device__ __forceinline__ int wave_min(int v) {
  v = min(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false));  // row_ror:4
  v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false));  // row_ror:8
  v = min(v, __shfl_xor(v, 16));
  v = min(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false));
  v = max(v, __shfl_xor(v, 16));
  v = max(v, __shfl_xor(v, 32));
  return v;
}

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
// Key pooling.  grid (pool.count, BH), 256 threads.
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
    const size_t out = (static_cast<size_t>(bh) * g.count + b) * D + dd;
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
  Hout[idx] = static_cast<float>(Hd);
  lvout[idx] = static_cast<int16_t>(kf);
}

// bf16 inputs.  grid (ceil(N/256), BH), 256 threads: 4 waves x 64 queries.
// Pooled keys stream through LDS in chunks of 32 rows; each chunk gives a
// 32(keys) x 32(queries) score block per MFMA column block, lane = query.
template <int D>
__global__ __launch_bounds__(256) void entropy_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kbar,
    const float* __restrict__ pool_w, int N, int NP, EntropyArgs ea, float* __restrict__ Hout,
    int16_t* __restrict__ lvout) {
  constexpr int NCH = D / 8;
  constexpr int KS = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t kb_lds[32 * D];
  __shared__ __attribute__((aligned(16))) float w_lds[32];
  const int bh = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int qbase = blockIdx.x * 256 + wave * 64;

  bf16x8 qf[2][KS];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int n = min(qbase + cb * 32 + col, N - 1);
    const uint16_t* p = q + (static_cast<size_t>(bh) * N + n) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[cb][ks] = *reinterpret_cast<const bf16x8*>(p + 16 * ks + 8 * h);
  }
  const uint16_t* kb = kbar + static_cast<size_t>(bh) * NP * D;
  const float c1 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  float m[2] = {TRA_NEG_INF, TRA_NEG_INF}, A[2] = {0.f, 0.f}, Bm[2] = {0.f, 0.f};

  const int nchunks = (NP + 31) / 32;
  for (int ci = 0; ci < nchunks; ++ci) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < 32 * NCH; idx += 256) {
      const int r = idx / NCH, c = idx % NCH;
      const int rowi = ci * 32 + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (rowi < NP) v = *reinterpret_cast<const uint4*>(kb + static_cast<size_t>(rowi) * D + c * 8);
      *reinterpret_cast<uint4*>(&kb_lds[r * D + ((c ^ swz<NCH>(r)) << 3)]) = v;
    }
    if (threadIdx.x < 32) {
      const int rowi = ci * 32 + threadIdx.x;
      w_lds[threadIdx.x] = rowi < NP ? pool_w[rowi] : 0.f;
    }
    __syncthreads();
    bf16x8 af[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      af[ks] = *reinterpret_cast<const bf16x8*>(&kb_lds[col * D + (((2 * ks + h) ^ swz<NCH>(col)) << 3)]);
    float w[16];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float4 w4 = *reinterpret_cast<const float4*>(&w_lds[8 * a + 4 * h]);
      w[4 * a + 0] = w4.x; w[4 * a + 1] = w4.y; w[4 * a + 2] = w4.z; w[4 * a + 3] = w4.w;
    }
    const bool partial = (ci + 1) * 32 > NP;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      f32x16 acc = {0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], qf[cb][ks], acc, 0, 0, 0);
      if (partial) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 8 * (i >> 2) + 4 * h + (i & 3);
          if (ci * 32 + r >= NP) acc[i] = TRA_NEG_INF;
        }
      }
      float mx = acc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, acc[i]);
      const float mnew = fmaxf(m[cb], mx * c1);
      if (mnew != TRA_NEG_INF) {
        float sA = 0.f, sB = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float t = fmaf(acc[i], c1, -mnew);
          const float e = __builtin_amdgcn_exp2f(t) * w[i];
          sA += e;
          sB = fmaf(e, t, sB);
        }
        if (A[cb] > 0.f) {
          const float alpha = __builtin_amdgcn_exp2f(m[cb] - mnew);
          Bm[cb] = alpha * fmaf(m[cb] - mnew, A[cb], Bm[cb]) + sB;
          A[cb] = fmaf(A[cb], alpha, sA);
        } else {
          Bm[cb] = sB;
          A[cb] = sA;
        }
        m[cb] = mnew;
      }
    }
  }
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float mp = __shfl_xor(m[cb], 32), Ap = __shfl_xor(A[cb], 32), Bp = __shfl_xor(Bm[cb], 32);
    const int n = qbase + cb * 32 + col;
    if (h == 0 && n < N) {
      const double M = fmax(static_cast<double>(m[cb]), static_cast<double>(mp));
      double At = 0.0, Bt = 0.0;
      if (A[cb] > 0.f) {
        const double s0 = exp2(static_cast<double>(m[cb]) - M);
        At += s0 * A[cb];
        Bt += s0 * (static_cast<double>(Bm[cb]) + (static_cast<double>(m[cb]) - M) * A[cb]);
      }
      if (Ap > 0.f) {
        const double s1 = exp2(static_cast<double>(mp) - M);
        At += s1 * Ap;
        Bt += s1 * (static_cast<double>(Bp) + (static_cast<double>(mp) - M) * Ap);
      }
      const double Hd = log(At) - 0.6931471805599453 * Bt / At;
      entropy_store(Hd, ea, static_cast<size_t>(bh) * N + n, Hout, lvout);
    }
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
// Tile lists.  One wave per query tile, lane = query (tile-local row-major).
// For every key frame within the wave's largest active temporal distance and
// every key-tile row the disks reach, each lane's footprint is a run of key-tile
// columns that contains the query tile's own column, so the union over the
// wave is the run [min lo, max hi].
// grid (ceil(tiles.count/4), BH), 256 threads.
// ---------------------------------------------------------------------------
template <bool FILL>
__global__ __launch_bounds__(256) void csr_kernel(const int16_t* __restrict__ lv,
                                                 const int32_t* __restrict__ r2,
                                                 const int32_t* __restrict__ dmax, int T,
                                                 int row_base, Grid g, int tw_shift,
                                                 int32_t* __restrict__ counts,
                                                 const int32_t* __restrict__ row_ptr,
                                                 int32_t* __restrict__ col_idx) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile = blockIdx.x * 4 + wave;
  if (tile >= g.count) return;  // wave-uniform
  const int bh = blockIdx.y;
  const size_t N = static_cast<size_t>(g.T) * g.H * g.W;
  const int64_t row = static_cast<int64_t>(bh) * g.count + tile;
  const int tq = tile / g.per_frame, rem = tile % g.per_frame;
  const int hq = (rem / g.nw) * g.th + (lane >> tw_shift);
  const int wq = (rem % g.nw) * g.tw + (lane & (g.tw - 1));
  const bool valid = hq < g.H && wq < g.W;
  int trow = 0, dm = -1;
  if (valid) {
    trow = lv[static_cast<size_t>(bh) * N + (static_cast<size_t>(tq) * g.H + hq) * g.W + wq] - row_base;
    dm = dmax[trow];
  }
  const int dmw = wave_max(dm);
  int count = 0;
  int out = FILL ? row_ptr[row] : 0;
  const int t_lo = max(0, tq - dmw), t_hi = min(T - 1, tq + dmw);
  for (int tk = t_lo; tk <= t_hi; ++tk) {
    const int delta = tk > tq ? tk - tq : tq - tk;
    const int thr = (valid && delta <= dm) ? r2[trow * T + delta] : -1;
    const int rad = thr >= 0 ? isqrt_i(thr) : -1;
    const int top = thr >= 0 ? max(0, hq - rad) : 0x7fffffff;
    const int bot = thr >= 0 ? min(g.H - 1, hq + rad) : -1;
    const int TOP = wave_min(top), BOT = wave_max(bot);
    if (BOT < TOP) continue;
    for (int tr = TOP / g.th; tr <= BOT / g.th; ++tr) {
      const int r0 = tr * g.th, r1 = min(g.H, r0 + g.th) - 1;
      const int dh = max(0, max(r0 - hq, hq - r1));
      const int remv = thr - dh * dh;
      int lo = 0x7fffffff, hi = -1;
      if (thr >= 0 && remv >= 0) {
        const int a = isqrt_i(remv);
        lo = max(0, wq - a) >> tw_shift;
        hi = min(g.W - 1, wq + a) >> tw_shift;
      }
      const int LO = wave_min(lo), HI = wave_max(hi);
      if (HI >= LO) {
        if constexpr (FILL) {
          const int base = (tk * g.nh + tr) * g.nw;
          for (int c = LO + lane; c <= HI; c += 64) col_idx[out + (c - LO)] = base + c;
          out += HI - LO + 1;
        } else {
          count += HI - LO + 1;
        }
      }
    }
  }
  if (!FILL && lane == 0) counts[row] = count;
}

// Exclusive scan of per-row counts.  One workgroup of 1024 threads.
// totals[0] = nnz, totals[1] = longest row, totals[2] = 1 if nnz >= 2^31.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ counts,
                                                   int64_t n, int32_t* __restrict__ row_ptr,
                                                   int64_t* __restrict__ totals) {
  __shared__ long long part[1024];
  __shared__ int pmax[1024];
  const int tid = threadIdx.x;
  const int64_t per = (n + 1023) / 1024;
  const int64_t b = tid * per, e = min(n, b + per);
  long long s = 0;
  int mx = 0;
  for (int64_t i = b; i < e; ++i) {
    s += counts[i];
    mx = max(mx, counts[i]);
  }
  part[tid] = s;
  pmax[tid] = mx;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    long long v = tid >= off ? part[tid - off] : 0;
    int vm = tid >= off ? pmax[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    pmax[tid] = max(pmax[tid], vm);
    __syncthreads();
  }
  long long run = part[tid] - s;  // exclusive prefix of this thread's chunk
  for (int64_t i = b; i < e; ++i) {
    row_ptr[i] = static_cast<int32_t>(run);
    run += counts[i];
  }
  if (tid == 1023) {
    row_ptr[n] = static_cast<int32_t>(part[1023]);
    totals[0] = part[1023];
    totals[1] = pmax[1023];
    totals[2] = part[1023] >= 0x7fffffffLL ? 1 : 0;
  }
}

// ---------------------------------------------------------------------------
// Block-sparse attention, bf16, 8x8 tiles.  One workgroup (2 waves) per query
// tile; wave w owns tile rows 4w..4w+3 (32 queries), lane%32 = query.
//   S^T (keys x queries) = K Q^T :  A = K rows from LDS, B = Q^T in registers
//   O^T (d x queries) += V^T P^T :  A = V^T via ds_read_b64_tr_b16, B = P^T
// The 32x32 output layout puts key rows {8(i/4) + 4(lane/32) + i%4} of a
// 32-key block in register i of a lane, which is exactly the k-slot order of
// the next MFMA's B operand, so P never leaves registers.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, const int16_t* __restrict__ lv,
    const int32_t* __restrict__ r2, int row_base, int T, Grid g,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx) {
  constexpr int NCH = D / 8;   // 16-byte chunks per key row
  constexpr int KS = D / 16;   // k-steps of S^T
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[64 * D];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int row = blockIdx.x;
  const int bh = row / g.count, tile = row % g.count;
  const size_t N = static_cast<size_t>(g.T) * g.H * g.W;
  const int tq = tile / g.per_frame, trem = tile % g.per_frame;
  const int h0 = (trem / g.nw) * 8, w0 = (trem % g.nw) * 8;
  const int mq = wave * 32 + col;
  const int hq = h0 + (mq >> 3), wq = w0 + (mq & 7);
  const bool qvalid = hq < g.H && wq < g.W;
  const size_t nq = (static_cast<size_t>(tq) * g.H + (qvalid ? hq : h0)) * g.W + (qvalid ? wq : w0);

  bf16x8 qf[KS];
  {
    const uint16_t* qp = q + (static_cast<size_t>(bh) * N + nq) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * h);
  }
  const int trow = qvalid ? lv[static_cast<size_t>(bh) * N + nq] - row_base : 0;
  const int32_t* r2row = r2 + trow * T;

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = (f32x16){0.f};
  float mref = TRA_NEG_INF, lsum = 0.f;
  const float c1 = 1.4426950408889634f / sqrtf(static_cast<float>(D));

  const uint16_t* kbase = k + static_cast<size_t>(bh) * N * D;
  const uint16_t* vbase = v + static_cast<size_t>(bh) * N * D;
  const int beg = row_ptr[row], end = row_ptr[row + 1];

  // Transposed-read addressing (per lane, fixed): group g4 of 16 lanes, lane
  // r4 = (lane%16)/4 picks the key row, j4 = lane%4 the 4-column slice.
  const int g4 = lane >> 4, r4 = (lane & 15) >> 2, j4 = lane & 3;

  for (int e = beg; e < end; ++e) {
    const int kt = col_idx[e];
    const int tk = kt / g.per_frame, krem = kt % g.per_frame;
    const int kr0 = (krem / g.nw) * 8, kc0 = (krem % g.nw) * 8;
    __syncthreads();
#pragma unroll
    for (int it = 0; it < (64 * NCH) / 128; ++it) {
      const int idx = threadIdx.x + it * 128;
      const int kk = idx / NCH, c = idx % NCH;
      const int kr = min(kr0 + (kk >> 3), g.H - 1), kc = min(kc0 + (kk & 7), g.W - 1);
      const size_t nk = (static_cast<size_t>(tk) * g.H + kr) * g.W + kc;
      const uint4 kv = *reinterpret_cast<const uint4*>(kbase + nk * D + c * 8);
      const uint4 vv = *reinterpret_cast<const uint4*>(vbase + nk * D + c * 8);
      const int off = kk * D + ((c ^ swz<NCH>(kk)) << 3);
      *reinterpret_cast<uint4*>(&k_lds[off]) = kv;
      *reinterpret_cast<uint4*>(&v_lds[off]) = vv;
    }
    __syncthreads();

    // Exact mask: key (kr0 + 4*blk + a, kc0 + 4*h + b) for register i = 4a + b.
    const int delta = tk > tq ? tk - tq : tq - tk;
    const int thr = qvalid ? r2row[delta] : -1;
    int remr[2][4], dw2[4];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int kr = kr0 + 4 * blk + a, dh = hq - kr;
        remr[blk][a] = (kr < g.H && thr >= 0) ? thr - dh * dh : -1;
      }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int kc = kc0 + 4 * h + b, dw = wq - kc;
      dw2[b] = kc < g.W ? dw * dw : 0x3fffffff;
    }
    const int mindw = min(min(dw2[0], dw2[1]), min(dw2[2], dw2[3]));
    const int maxdw = max(max(dw2[0], dw2[1]), max(dw2[2], dw2[3]));
    bool doblk[2], fullblk[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int mxr = max(max(remr[blk][0], remr[blk][1]), max(remr[blk][2], remr[blk][3]));
      const int mnr = min(min(remr[blk][0], remr[blk][1]), min(remr[blk][2], remr[blk][3]));
      doblk[blk] = __any(mxr >= mindw);
      fullblk[blk] = __all(mnr >= maxdw);
    }
    if (!doblk[0] && !doblk[1]) continue;

    f32x16 sacc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      sacc[blk] = (f32x16){0.f};
      if (!doblk[blk]) continue;
      const int kk = 32 * blk + col;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 af =
            *reinterpret_cast<const bf16x8*>(&k_lds[kk * D + (((2 * ks + h) ^ swz<NCH>(kk)) << 3)]);
        sacc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[ks], sacc[blk], 0, 0, 0);
      }
      if (!fullblk[blk]) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (dw2[i & 3] > remr[blk][i >> 2]) sacc[blk][i] = TRA_NEG_INF;
      }
    }

    float mx = TRA_NEG_INF;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
      if (doblk[blk]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[blk][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mcand = mx * c1;
    // Lazy rescale: the reference max moves only when a score exceeds it by
    // more than 2^8, so probabilities stay <= 256 between rescales.
    if (__any(mcand > mref + 8.f)) {
      const float mn = fmaxf(mref, mcand);
      const float alpha = mref == TRA_NEG_INF ? 0.f : __builtin_amdgcn_exp2f(mref - mn);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      mref = mn;
    }
    const float msub = mref == TRA_NEG_INF ? 0.f : mref;

#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      if (!doblk[blk]) continue;
      bf16x8 pf[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[blk][8 * j + 2 * x], c1, -msub));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[blk][8 * j + 2 * x + 1], c1, -msub));
          lsum += p0 + p1;
          const bf16x2 pp = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
          pf[j][2 * x] = pp[0];
          pf[j][2 * x + 1] = pp[1];
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          bf16x8 vf;
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const int kr = 32 * blk + 16 * j + 8 * s + 4 * (g4 >> 1) + r4;
            const int d = 32 * db + 16 * (g4 & 1) + 4 * j4;
            const int off = kr * D + ((((d >> 3)) ^ swz<NCH>(kr)) << 3) + (d & 7);
            const bf16x4 t4 = lds_read_tr(v_lds, off);
            vf[4 * s + 0] = t4[0];
            vf[4 * s + 1] = t4[1];
            vf[4 * s + 2] = t4[2];
            vf[4 * s + 3] = t4[3];
          }
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[j], oacc[db], 0, 0, 0);
        }
      }
    }
  }

  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (qvalid) {
    uint16_t* op = o + (static_cast<size_t>(bh) * N + nq) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = 32 * db + 8 * a + 4 * h;
        const bf16x2 lo2 = __builtin_convertvector(
            ((f32x2){oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv}), bf16x2);
        const bf16x2 hi2 = __builtin_convertvector(
            ((f32x2){oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv}), bf16x2);
        const bf16x4 out4 = {lo2[0], lo2[1], hi2[0], hi2[1]};
        *reinterpret_cast<bf16x4*>(op + d0) = out4;
      }
  }
}

// fp32 inputs: one thread per query, K/V tiles in LDS, fp32 online softmax.
template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, const int16_t* __restrict__ lv, const int32_t* __restrict__ r2,
    int row_base, int T, Grid g, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx) {
  __shared__ float k_lds[64][D];
  __shared__ float v_lds[64][D];
  const int lane = threadIdx.x;
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
  const int beg = row_ptr[row], end = row_ptr[row + 1];
  for (int e = beg; e < end; ++e) {
    const int kt = col_idx[e];
    const int tk = kt / g.per_frame, krem = kt % g.per_frame;
    const int kr0 = (krem / g.nw) * 8, kc0 = (krem % g.nw) * 8;
    __syncthreads();
    for (int idx = lane; idx < 64 * D / 4; idx += 64) {
      const int kk = idx / (D / 4), c = idx % (D / 4);
      const int kr = min(kr0 + (kk >> 3), g.H - 1), kc = min(kc0 + (kk & 7), g.W - 1);
      const size_t nk = (static_cast<size_t>(tk) * g.H + kr) * g.W + kc;
      *reinterpret_cast<float4*>(&k_lds[kk][4 * c]) = *reinterpret_cast<const float4*>(kbase + nk * D + 4 * c);
      *reinterpret_cast<float4*>(&v_lds[kk][4 * c]) = *reinterpret_cast<const float4*>(vbase + nk * D + 4 * c);
    }
    __syncthreads();
    const int delta = tk > tq ? tk - tq : tq - tk;
    const int thr = qvalid ? r2row[delta] : -1;
    for (int kk = 0; kk < 64; ++kk) {
      const int kr = kr0 + (kk >> 3), kc = kc0 + (kk & 7);
      const int dh = hq - kr, dw = wq - kc;
      if (kr >= g.H || kc >= g.W || thr < 0 || dh * dh + dw * dw > thr) continue;
      float s = 0.f;
#pragma unroll
      for (int dd = 0; dd < D; ++dd) s = fmaf(qr[dd], k_lds[kk][dd], s);
      s *= scale;
      if (s > mref) {
        const float alpha = expf(mref - s);
        lsum *= alpha;
#pragma unroll
        for (int dd = 0; dd < D; ++dd) acc[dd] *= alpha;
        mref = s;
      }
      const float p = expf(s - mref);
      lsum += p;
#pragma unroll
      for (int dd = 0; dd < D; ++dd) acc[dd] = fmaf(p, v_lds[kk][dd], acc[dd]);
    }
  }
  if (qvalid) {
    float* op = o + (static_cast<size_t>(bh) * N + nq) * D;
    const float inv = 1.f / lsum;
#pragma unroll
    for (int dd = 0; dd < D; ++dd) op[dd] = acc[dd] * inv;
  }
}

// ---------------------------------------------------------------------------
// Exact pair counts.
// ---------------------------------------------------------------------------
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
    for (int tk = 0; tk < T; ++tk) {
      const int thr = row[tk > t ? tk - t : t - tk];
      if (thr < 0) continue;
      const int rad = isqrt_i(thr);
      for (int hk = max(0, hh - rad); hk <= min(g.H - 1, hh + rad); ++hk) {
        const int a = isqrt_i(thr - (hk - hh) * (hk - hh));
        cnt += min(g.W - 1, ww + a) - max(0, ww - a) + 1;
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
                          int BH, int N, int n_pool, const EntropyArgs& ea, float* H_out,
                          int16_t* lv_out, hipStream_t s) {
  const dim3 grid((N + 255) / 256, BH), block(256);
  if (dtype == 1) {
    const auto* qq = static_cast<const uint16_t*>(q);
    const auto* kb = static_cast<const uint16_t*>(kbar);
    if (d == 128) entropy_bf16_kernel<128><<<grid, block, 0, s>>>(qq, kb, pool_w, N, n_pool, ea, H_out, lv_out);
    else entropy_bf16_kernel<64><<<grid, block, 0, s>>>(qq, kb, pool_w, N, n_pool, ea, H_out, lv_out);
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

hipError_t launch_csr_count(const int16_t* lv, const int32_t* r2, const int32_t* dmax, int T,
                            int row_base, int BH, const Grid& tiles, int32_t* counts,
                            hipStream_t s) {
  const dim3 grid((tiles.count + 3) / 4, BH), block(256);
  csr_kernel<false><<<grid, block, 0, s>>>(lv, r2, dmax, T, row_base, tiles, log2i(tiles.tw),
                                           counts, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_scan(const int32_t* counts, int64_t n_rows, int32_t* row_ptr, int64_t* totals,
                       hipStream_t s) {
  scan_kernel<<<1, 1024, 0, s>>>(counts, n_rows, row_ptr, totals);
  return hipGetLastError();
}

hipError_t launch_csr_fill(const int16_t* lv, const int32_t* r2, const int32_t* dmax, int T,
                           int row_base, int BH, const Grid& tiles, const int32_t* row_ptr,
                           int32_t* col_idx, hipStream_t s) {
  const dim3 grid((tiles.count + 3) / 4, BH), block(256);
  csr_kernel<true><<<grid, block, 0, s>>>(lv, r2, dmax, T, row_base, tiles, log2i(tiles.tw),
                                          nullptr, row_ptr, col_idx);
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, int d, const void* q, const void* k, const void* v,
                            void* o, const int16_t* lv, const int32_t* r2, int row_base,
                            int BH, const Grid& tiles, const int32_t* row_ptr,
                            const int32_t* col_idx, hipStream_t s) {
  const unsigned rows = static_cast<unsigned>(BH) * tiles.count;
  if (dtype == 1) {
    const auto* qq = static_cast<const uint16_t*>(q);
    const auto* kk = static_cast<const uint16_t*>(k);
    const auto* vv = static_cast<const uint16_t*>(v);
    auto* oo = static_cast<uint16_t*>(o);
    if (d == 128)
      attn_bf16_kernel<128><<<rows, 128, 0, s>>>(qq, kk, vv, oo, lv, r2, row_base, tiles.T, tiles, row_ptr, col_idx);
    else
      attn_bf16_kernel<64><<<rows, 128, 0, s>>>(qq, kk, vv, oo, lv, r2, row_base, tiles.T, tiles, row_ptr, col_idx);
  } else {
    const auto* qq = static_cast<const float*>(q);
    const auto* kk = static_cast<const float*>(k);
    const auto* vv = static_cast<const float*>(v);
    auto* oo = static_cast<float*>(o);
    if (d == 128)
      attn_f32_kernel<128><<<rows, 64, 0, s>>>(qq, kk, vv, oo, lv, r2, row_base, tiles.T, tiles, row_ptr, col_idx);
    else
      attn_f32_kernel<64><<<rows, 64, 0, s>>>(qq, kk, vv, oo, lv, r2, row_base, tiles.T, tiles, row_ptr, col_idx);
  }
  return hipGetLastError();
}

hipError_t launch_stats(const int16_t* lv, const int32_t* r2, int T, int row_base, int BH,
                        const Grid& tiles, const int32_t* row_ptr, const int32_t* col_idx,
                        unsigned long long* out2, hipStream_t s) {
  const int64_t nq = static_cast<int64_t>(BH) * tiles.T * tiles.H * tiles.W;
  retained_kernel<<<static_cast<unsigned>((nq + 255) / 256), 256, 0, s>>>(lv, r2, T, row_base, tiles, nq, out2);
  const int64_t nr = static_cast<int64_t>(BH) * tiles.count;
  listed_kernel<<<static_cast<unsigned>((nr + 255) / 256), 256, 0, s>>>(tiles, nr, row_ptr, col_idx, out2 + 1);
  return hipGetLastError();
}

}  // namespace tra
