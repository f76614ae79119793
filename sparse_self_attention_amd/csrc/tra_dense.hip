// Dense warm-up pass of the Token Radius Attention pipeline for gfx950.
//
// "Token Radius Attention for Efficient Video Generation" (summary page,
// section 2, "Le Pipeline TRA"): during dense warm-up steps the full attention
// is computed and each query's attention entropy is recorded; the entropies
// then set the budgets of the sparse steps that follow.  This file computes
// both in one pass: softmax(Q K^T / sqrt(d)) V over all N keys of a head and,
// alongside the online softmax, the entropy
//     H_i = ln l_i - ln2 * (sum_j p_ij t_ij) / l_i,
// with t_ij = s_ij*log2(e) - m_i (m_i the running reference, log2 units),
// p_ij = 2^t_ij and l_i = sum_j p_ij.  The second sum costs one fused
// multiply-add per score; the reference's moves rescale it like l.
//
// Kernels:
//   dense_bf16_kernel    8 waves x 32 queries share each 64-key tile of K and V,
//                        streamed into LDS by range-checked buffer DMA one tile
//                        ahead; S^T = K Q^T and O^T += V^T P^T on 32x32x16 bf16
//                        MFMA (the layout of the block-sparse kernel, without
//                        masks and tile lists).  fp32 softmax; the entropy sums
//                        are taken in fp32 per 16-key half block and carried in
//                        fp64 across blocks.
//   dense_f32_kernel     fp32 inputs: one thread per query, fp64 scores.
//   levels_from_entropy  budget level of each query from a given entropy.
#include "tra_internal.h"
#include "tra_device.h"

#include <math.h>

#include <algorithm>

namespace tra {

namespace {

// LDS row strides of the staged tiles (bytes): the padded layouts of the
// block-sparse kernel (conflict-free 16-byte operand reads of K rows and
// transposing 8-byte reads of V rows).
template <int D> struct DenseLds {
  static constexpr int KSTR = 2 * D + 16;
  static constexpr int VSTR = 2 * D + 64;
  static constexpr int KSEG = 64 * KSTR / 1024;
  static constexpr int VSEG = 64 * VSTR / 1024;
  static constexpr int BUF = (KSEG + VSEG) * 1024;
  static_assert(64 * KSTR % 1024 == 0 && 64 * VSTR % 1024 == 0, "tile must be whole segments");
};

constexpr int DENSE_WAVES = 8;
constexpr int DENSE_QB = 32 * DENSE_WAVES;  // queries per workgroup

}  // namespace

// grid: ceil(groups / 8) * 8 workgroups of 512 threads, groups = BH * ceil(N / 256).
template <int D, bool ENT>
__global__ __launch_bounds__(512) void dense_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ Hout, int N, int qblocks, int n_groups) {
  using L = DenseLds<D>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  __shared__ __attribute__((aligned(1024))) char kv0[L::BUF];
  __shared__ __attribute__((aligned(1024))) char kv1[L::BUF];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, col = lane & 31;
  // Consecutive query blocks of a head go to the same XCD (dispatch is
  // round-robin over the 8 XCDs), so the blocks resident on one XCD stream
  // the same K/V tiles through its L2.
  const int per_xcd = gridDim.x / 8;
  const int gid = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (gid >= n_groups) return;  // uniform over the workgroup, before any barrier
  const int bh = gid / qblocks;
  const int n = (gid % qblocks) * DENSE_QB + wave * 32 + col;
  const bool qvalid = n < N;
  const size_t head = static_cast<size_t>(bh) * N;

  bf16x8 qf[KS];
  {
    const uint16_t* qp = q + (head + min(n, N - 1)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * h);
  }

  // Tile e holds keys 64e .. 64e+63 (contiguous rows of the head).  Keys past
  // the head's end read as zero through the range check and are masked.
  const i32x4 krsrc = make_rsrc(k + head * D, static_cast<uint32_t>(static_cast<size_t>(N) * D * 2));
  const i32x4 vrsrc = make_rsrc(v + head * D, static_cast<uint32_t>(static_cast<size_t>(N) * D * 2));
  // DMA segment s (1 KB) of a tile: lane l's 16 bytes land at s*1KB + 16*l,
  // the (key row, chunk) that the padded layout puts there; wave w issues
  // segments w, w + 8, w + 16, ... (pad chunks re-fetch the row's chunk 0).
  constexpr int NK = (L::KSEG + DENSE_WAVES - 1) / DENSE_WAVES;
  constexpr int NV = (L::VSEG + DENSE_WAVES - 1) / DENSE_WAVES;
  auto seg_off = [&](int stride, int seg) {
    const int ob = seg * 1024 + lane * 16;
    const int kk = ob / stride;
    const int c = (ob % stride) / 16;
    return static_cast<uint32_t>(kk * D * 2 + (c < D / 8 ? c : 0) * 16);
  };
  uint32_t koff[NK], voff[NV];
#pragma unroll
  for (int i = 0; i < NK; ++i) koff[i] = seg_off(L::KSTR, min(wave + DENSE_WAVES * i, L::KSEG - 1));
#pragma unroll
  for (int i = 0; i < NV; ++i) voff[i] = seg_off(L::VSTR, min(wave + DENSE_WAVES * i, L::VSEG - 1));
  auto lds_addr = [&](const char* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p)));
  };
  auto issue = [&](int e, char* buf) {
    const uint32_t tile_bytes = static_cast<uint32_t>(e) * 64u * (D * 2u);
    const uint32_t kb = lds_addr(buf), vb = lds_addr(buf + L::KSEG * 1024);
#pragma unroll
    for (int i = 0; i < NK; ++i)
      if (wave + DENSE_WAVES * i < L::KSEG)
        lds_dma16_buf(krsrc, tile_bytes + koff[i],
                      __builtin_amdgcn_readfirstlane(kb + (wave + DENSE_WAVES * i) * 1024));
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (wave + DENSE_WAVES * i < L::VSEG)
        lds_dma16_buf(vrsrc, tile_bytes + voff[i],
                      __builtin_amdgcn_readfirstlane(vb + (wave + DENSE_WAVES * i) * 1024));
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = (f32x16){0.f};
  float lsum = 0.f;            // without entropy: sum of the bf16 probabilities used by PV
  double lsum_d = 0.0, bsum_d = 0.0;  // with entropy: sum p and sum p*t, this lane's keys
  const float c1 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  const int g4 = lane >> 4, r4 = (lane & 15) >> 2, j4 = lane & 3;
  const int kread = col * L::KSTR + h * 16;
  const int vread = (4 * (g4 >> 1) + r4) * L::VSTR + (16 * (g4 & 1) + 4 * j4) * 2;
  const int partner = (lane ^ 32) << 2;
  // The softmax reference (log2 units) starts at the query's score with its
  // own key, which the pass visits like every other key, so it is finite from
  // the start.  Each lane of a query pair holds half of the dot product.
  float mref;
  {
    const uint16_t* kp = k + (head + min(n, N - 1)) * D;
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
    dot += __int_as_float(__builtin_amdgcn_ds_bpermute(partner, __float_as_int(dot)));
    mref = dot * c1;
  }

  auto scores = [&](const char* buf, int blk) {
    f32x16 acc = (f32x16){0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(buf + kread + 32 * blk * L::KSTR + 32 * ks);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[ks], acc, 0, 0, 0);
    }
    return acc;
  };
  auto rowmax = [&](const f32x16& s) {
    float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, s[i]), s[i + 1]);
    return fmaxf(mx, s[15]);
  };
  // Probabilities against the current reference (lazy rescale: the reference
  // moves only when a lane's probabilities of a block, formed against it, sum
  // to more than 2^10, so between moves every probability is <= 2^10).
  auto probs = [&](const f32x16& s, bf16x8* pf, float* ls, float* bs) {
    const float msub = mref;
    const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
    float l2[2] = {0.f, 0.f}, b2[2] = {0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t pk[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float t0 = fmaf(s[8 * j + 2 * x], c1, -msub);
        const float t1 = fmaf(s[8 * j + 2 * x + 1], c1, -msub);
        const float p0 = __builtin_amdgcn_exp2f(t0);
        const float p1 = __builtin_amdgcn_exp2f(t1);
        pk[x] = pack_bf16x2(p0, p1);
        if constexpr (ENT) {
          l2[j] += p0 + p1;
          b2[j] = fmaf(p1, t1, fmaf(p0, t0, b2[j]));
        } else {
          l2[j] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[x]), ones, l2[j], false);
        }
      }
      pf[j] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
    }
    *ls = l2[0] + l2[1];
    *bs = b2[0] + b2[1];
  };
  auto softmax = [&](const f32x16& s, bf16x8* pf) {
    float ls, bs;
    probs(s, pf, &ls, &bs);
    if (__any(!(ls <= 1024.f))) {
      float mx = rowmax(s);
      mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_bpermute(partner, __float_as_int(mx))));
      if (__any(mx * c1 > mref)) {
        const float mn = fmaxf(mref, mx * c1);
        const float alpha = __builtin_amdgcn_exp2f(mref - mn);
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        if constexpr (ENT) {
          // t moves by (mref - mn): sum p*t -> alpha * (sum p*t + (mref - mn) * sum p).
          const double ad = static_cast<double>(alpha);
          bsum_d = ad * (bsum_d + static_cast<double>(mref - mn) * lsum_d);
          lsum_d *= ad;
        } else {
          lsum *= alpha;
        }
        mref = mn;
        probs(s, pf, &ls, &bs);
      }
    }
    if constexpr (ENT) {
      lsum_d += static_cast<double>(ls);
      bsum_d += static_cast<double>(bs);
    } else {
      lsum += ls;
    }
  };
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
  // Keys past the head's end: a finite sentinel score, so that p = 0 and
  // p * t = 0 exactly.
  auto mask_tail = [&](f32x16& s, int key0) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (key0 + 8 * (i >> 2) + 4 * h + (i & 3) >= N) s[i] = -3.0e38f;
  };
  auto compute = [&](int e, const char* buf, bool more, char* nbuf) {
    f32x16 s0 = scores(buf, 0);
    f32x16 s1 = scores(buf, 1);
    if (more) issue(e + 1, nbuf);
    if ((e + 1) * 64 > N) {  // the last, partial tile (uniform)
      mask_tail(s0, 64 * e);
      mask_tail(s1, 64 * e + 32);
    }
    bf16x8 pf0[2], pf1[2];
    softmax(s0, pf0);
    pv(buf, 0, pf0);
    softmax(s1, pf1);
    pv(buf, 1, pf1);
  };

  // One barrier per tile; tile e+1 streams into the other buffer while e is
  // consumed (the scheme of the block-sparse kernel).
  const int n_tiles = (N + 63) / 64;
  issue(0, kv0);
  for (int e = 0;;) {
    wait_vmcnt<0>();
    lds_barrier();
    compute(e, kv0, e + 1 < n_tiles, kv1);
    if (++e == n_tiles) break;
    wait_vmcnt<0>();
    lds_barrier();
    compute(e, kv1, e + 1 < n_tiles, kv0);
    if (++e == n_tiles) break;
  }

  float inv;
  if constexpr (ENT) {
    const double lt = lsum_d + __shfl_xor(lsum_d, 32), bt = bsum_d + __shfl_xor(bsum_d, 32);
    inv = static_cast<float>(1.0 / lt);
    if (h == 0 && qvalid) Hout[head + n] = static_cast<float>(log(lt) - 0.6931471805599453 * bt / lt);
  } else {
    const float lt = lsum + __int_as_float(__builtin_amdgcn_ds_bpermute(partner, __float_as_int(lsum)));
    inv = 1.f / lt;
  }
  if (qvalid) {
    uint16_t* op = o + (head + n) * D;
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

// fp32 inputs: one thread per query; keys and values staged in LDS 64 at a
// time; fp64 scores (exact products of fp32 values) and fp64 softmax sums;
// fp32 output accumulator.  grid (ceil(N / 64), BH), 64 threads.
template <int D>
__global__ __launch_bounds__(64) void dense_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                       const float* __restrict__ v, float* __restrict__ o,
                                                       float* __restrict__ Hout, int N) {
  __shared__ float k_lds[64][D];
  __shared__ float v_lds[64][D];
  const int lane = threadIdx.x;
  const int bh = blockIdx.y;
  const int n = blockIdx.x * 64 + lane;
  const bool qvalid = n < N;
  const size_t head = static_cast<size_t>(bh) * N;
  float qr[D], acc[D];
  const float* qp = q + (head + min(n, N - 1)) * D;
#pragma unroll
  for (int dd = 0; dd < D; ++dd) {
    qr[dd] = qp[dd];
    acc[dd] = 0.f;
  }
  const double scale = 1.0 / sqrt(static_cast<double>(D));
  double m = -HUGE_VAL, l = 0.0, b = 0.0;  // b = sum p * (s - m)
  for (int j0 = 0; j0 < N; j0 += 64) {
    __syncthreads();
    for (int idx = lane; idx < 64 * D / 4; idx += 64) {
      const int kk = idx / (D / 4), c = idx % (D / 4);
      const size_t nk = head + min(j0 + kk, N - 1);
      *reinterpret_cast<float4*>(&k_lds[kk][4 * c]) = *reinterpret_cast<const float4*>(k + nk * D + 4 * c);
      *reinterpret_cast<float4*>(&v_lds[kk][4 * c]) = *reinterpret_cast<const float4*>(v + nk * D + 4 * c);
    }
    __syncthreads();
    const int cnt = min(64, N - j0);
    for (int kk = 0; kk < cnt; ++kk) {
      double s = 0.0;
#pragma unroll
      for (int dd = 0; dd < D; ++dd) s = fma(static_cast<double>(qr[dd]), static_cast<double>(k_lds[kk][dd]), s);
      s *= scale;
      if (s > m) {
        if (l > 0.0) {  // move the reference: every term so far scales by alpha
          const double alpha = exp(m - s);
          b = alpha * (b + (m - s) * l);
          l *= alpha;
          const float af = static_cast<float>(alpha);
#pragma unroll
          for (int dd = 0; dd < D; ++dd) acc[dd] *= af;
        }
        m = s;
      }
      const double t = s - m;
      const double p = exp(t);
      l += p;
      b = fma(p, t, b);
      const float pf = static_cast<float>(p);
#pragma unroll
      for (int dd = 0; dd < D; ++dd) acc[dd] = fmaf(pf, v_lds[kk][dd], acc[dd]);
    }
  }
  if (qvalid) {
    float* op = o + (head + n) * D;
    const float inv = static_cast<float>(1.0 / l);
#pragma unroll
    for (int dd = 0; dd < D; ++dd) op[dd] = acc[dd] * inv;
    if (Hout) Hout[head + n] = static_cast<float>(log(l) - b / l);
  }
}

// Budget level of each query from its entropy (fp64 arithmetic on the given
// fp32 value): k = clamp(floor(q_lv * (a*H + c)), k_lo, k_hi).  The entropy is
// copied into the plan's own buffer.
__global__ __launch_bounds__(256) void levels_from_entropy_kernel(const float* __restrict__ Hin, int64_t n,
                                                                  EntropyArgs ea, float* __restrict__ Hout,
                                                                  int16_t* __restrict__ lv) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) {
    const double Hd = static_cast<double>(Hin[i]);
    double kf = floor(static_cast<double>(ea.levels_per_nat) * (ea.a * Hd + ea.c));
    kf = fmin(fmax(kf, static_cast<double>(ea.k_lo)), static_cast<double>(ea.k_hi));
    Hout[i] = Hin[i];
    lv[i] = static_cast<int16_t>(kf);
  }
}

hipError_t launch_dense(int dtype, int d, const void* q, const void* k, const void* v, void* o,
                        float* H, int BH, int N, hipStream_t s) {
  if (dtype == 1) {
    const auto* qq = static_cast<const uint16_t*>(q);
    const auto* kk = static_cast<const uint16_t*>(k);
    const auto* vv = static_cast<const uint16_t*>(v);
    auto* oo = static_cast<uint16_t*>(o);
    const int qblocks = (N + DENSE_QB - 1) / DENSE_QB;
    const int64_t groups = static_cast<int64_t>(BH) * qblocks;
    const unsigned grid = static_cast<unsigned>((groups + 7) / 8 * 8);
    const int ng = static_cast<int>(groups);
#define TRA_DENSE(DD, E) dense_bf16_kernel<DD, E><<<grid, 512, 0, s>>>(qq, kk, vv, oo, H, N, qblocks, ng)
    if (H) {
      if (d == 128) TRA_DENSE(128, true);
      else TRA_DENSE(64, true);
    } else {
      if (d == 128) TRA_DENSE(128, false);
      else TRA_DENSE(64, false);
    }
#undef TRA_DENSE
  } else {
    const dim3 grid((N + 63) / 64, BH);
    const auto* qq = static_cast<const float*>(q);
    const auto* kk = static_cast<const float*>(k);
    const auto* vv = static_cast<const float*>(v);
    auto* oo = static_cast<float*>(o);
    if (d == 128) dense_f32_kernel<128><<<grid, 64, 0, s>>>(qq, kk, vv, oo, H, N);
    else dense_f32_kernel<64><<<grid, 64, 0, s>>>(qq, kk, vv, oo, H, N);
  }
  return hipGetLastError();
}

hipError_t launch_levels_from_entropy(const float* Hin, int64_t n, const EntropyArgs& ea, float* Hout,
                                      int16_t* lv, hipStream_t s) {
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 8192);
  levels_from_entropy_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(Hin, n, ea, Hout, lv);
  return hipGetLastError();
}

}  // namespace tra
