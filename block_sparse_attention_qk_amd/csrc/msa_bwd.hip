// Main Branch backward for gfx950: dQ, dK, dV of exact softmax GQA attention
// over the cached blocks (ai-beat "flash-msa-sparse-attention-training",
// paragraph 2: training needs a backward pass through the sparse pattern;
// keyed on the cached block indices, xcelit "How MSA works").
//
// KV-stationary schedule, one work item per (batch, group, block) and window.
// Each of the 4 waves owns 32 keys of the block: their K and V rows stay in
// registers as MFMA operands, their dK/dV accumulate in registers over all
// the pairs that read the block.  Tiles of 64 query rows (64/R tokens x R
// heads) are staged in LDS in row-major and transposed form.  Per tile:
//   S = Q K^T, dP = dO V^T           (rows along M, owned keys along N)
//   P = exp(scale S - LSE), dS = P (dP - D)
//   dV += P^T dO, dK += dS^T Q        (P, dS reused in place as A operands)
//   dQ^T = K^T dS^T                   (dS exchanged through LDS; each wave
//                                      makes a 16- or 32-wide slice of dQ)
// dQ leaves as one bf16 partial per (token, slot); a combine pass sums a
// token's partials.  dK/dV are added into fp32 accumulators once per item.
// Nothing is accumulated with atomics.
#include "msa_common.h"
#include "msa_internal.h"

#include <algorithm>

namespace msa {

template <int D, int R>
__global__ __launch_bounds__(256, 1) void k_bwd_kv(
    const bf16raw* __restrict__ q, const bf16raw* __restrict__ k, const bf16raw* __restrict__ v,
    const bf16raw* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dd,
    const int4* __restrict__ items, const int32_t* __restrict__ item_count, const int32_t* __restrict__ list,
    bf16raw* __restrict__ dq_part, float* __restrict__ dk_acc, float* __restrict__ dv_acc, int T, int H, int G,
    int K, int t0, int W, int max_items, float scale, float sl2) {
  constexpr int KS = D / 32;     // k-steps over the head dim
  constexpr int CT = D / 16;     // head-dim tiles
  constexpr int CW = D / 64;     // head-dim tiles of dQ made by each wave
  constexpr int TR = 64;         // query rows per tile
  constexpr int TT = TR / R;     // tokens per tile
  constexpr int LDQ = D + 8;     // row-major tile stride (bf16)
  constexpr int LDT = TR + 8;    // transposed tile stride (bf16)
  constexpr int LDS_ = BLK + 8;  // dS tile stride (bf16)
  __shared__ __attribute__((aligned(16))) bf16raw Qs[TR * LDQ];
  __shared__ __attribute__((aligned(16))) bf16raw dOs[TR * LDQ];
  __shared__ __attribute__((aligned(16))) bf16raw QsT[D * LDT];
  __shared__ __attribute__((aligned(16))) bf16raw dOsT[D * LDT];
  __shared__ __attribute__((aligned(16))) bf16raw dSs[TR * LDS_];
  __shared__ float lse_s[TR], dd_s[TR];
  __shared__ int tok_s[TR], pair_s[TR];

  const int bg = blockIdx.y;
  if ((int)blockIdx.x >= item_count[bg]) return;
  const int4 it = items[(size_t)bg * max_items + blockIdx.x];
  const int blk = it.x, start = it.y, len = it.z;
  const int b = bg / G, g = bg % G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, q4 = lane >> 4;
  const size_t kv0 = (size_t)(b * T + blk * BLK) * G + g;
  const size_t pair0 = (size_t)bg * W * K;
  const int32_t* lst = list + pair0 + start;
  const int kw = 32 * wave;            // first key owned by this wave
  const int cbase = 16 * CW * wave;    // first dQ column made by this wave

  bf16x8 bk[2][KS], bv[2][KS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const size_t rrow = (kv0 + (size_t)(kw + 16 * nt + l16) * G) * D + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bk[nt][ks] = ld8(k + rrow + 32 * ks);
      bv[nt][ks] = ld8(v + rrow + 32 * ks);
    }
  }
  // K^T slice (head-dim rows cbase.., all 128 keys in kperm slot order)
  bf16x8 akt[CW][4];
#pragma unroll
  for (int cw = 0; cw < CW; ++cw)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint32_t w[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        // slots e = 2m, 2m+1 hold keys of the kperm order (see msa_common.h)
        const int e0 = 2 * m, e1 = 2 * m + 1;
        const int k0 = 32 * ks + (e0 < 4 ? 4 * q4 + e0 : 16 + 4 * q4 + (e0 - 4));
        const int k1 = 32 * ks + (e1 < 4 ? 4 * q4 + e1 : 16 + 4 * q4 + (e1 - 4));
        const uint32_t lo = k[(kv0 + (size_t)k0 * G) * D + cbase + 16 * cw + l16];
        const uint32_t hi = k[(kv0 + (size_t)k1 * G) * D + cbase + 16 * cw + l16];
        w[m] = lo | (hi << 16);
      }
      akt[cw][ks] = as_bf8(make_uint4(w[0], w[1], w[2], w[3]));
    }

  f32x4 dka[2][CT], dva[2][CT];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) dka[nt][ct] = dva[nt][ct] = zero4();

  const int ntiles = (len + TT - 1) / TT;
  for (int tile = 0; tile < ntiles; ++tile) {
    // ---- stage rows: Q, dO (row-major and transposed), LSE, D
    if (threadIdx.x < TR) {
      const int row = threadIdx.x, li = tile * TT + row / R;
      const bool val = li < len;
      const int p = val ? lst[li] : -1;
      const int t = val ? t0 + p / K : -1;
      const size_t hrow = (size_t)(b * T + (val ? t : 0)) * H + g * R + row % R;
      tok_s[row] = t;
      pair_s[row] = p;
      lse_s[row] = val ? lse[hrow] * LOG2E : INFINITY;
      dd_s[row] = val ? Dd[hrow] : 0.f;
    }
    for (int u = threadIdx.x; u < (TR / 2) * (D / 8); u += 256) {
      const int rp = u & 31, cc = u >> 5;
      const int r0 = 2 * rp, r1 = r0 + 1;
      const int li0 = tile * TT + r0 / R, li1 = tile * TT + r1 / R;
      const bool v0 = li0 < len, v1 = li1 < len;
      const int t0r = v0 ? t0 + lst[li0] / K : 0, t1r = v1 ? t0 + lst[li1] / K : 0;
      const size_t a0 = ((size_t)(b * T + t0r) * H + g * R + r0 % R) * D + 8 * cc;
      const size_t a1 = ((size_t)(b * T + t1r) * H + g * R + r1 % R) * D + 8 * cc;
      const uint4 z = make_uint4(0u, 0u, 0u, 0u);
      const uint4 x0 = v0 ? ld16u(q + a0) : z, x1 = v1 ? ld16u(q + a1) : z;
      const uint4 y0 = v0 ? ld16u(dout + a0) : z, y1 = v1 ? ld16u(dout + a1) : z;
      st16u(&Qs[r0 * LDQ + 8 * cc], x0);
      st16u(&Qs[r1 * LDQ + 8 * cc], x1);
      st16u(&dOs[r0 * LDQ + 8 * cc], y0);
      st16u(&dOs[r1 * LDQ + 8 * cc], y1);
      const int pos = 32 * (r0 >> 5) + kperm(r0 & 31);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t a = word_of(x0, m), c = word_of(x1, m);
        const uint32_t e = word_of(y0, m), f = word_of(y1, m);
        *reinterpret_cast<uint32_t*>(&QsT[(8 * cc + 2 * m) * LDT + pos]) = pair_lo(a, c);
        *reinterpret_cast<uint32_t*>(&QsT[(8 * cc + 2 * m + 1) * LDT + pos]) = pair_hi(a, c);
        *reinterpret_cast<uint32_t*>(&dOsT[(8 * cc + 2 * m) * LDT + pos]) = pair_lo(e, f);
        *reinterpret_cast<uint32_t*>(&dOsT[(8 * cc + 2 * m + 1) * LDT + pos]) = pair_hi(e, f);
      }
    }
    __syncthreads();

    // ---- S = Q K^T and dP = dO V^T for the owned keys
    f32x4 sacc[4][2], pacc[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) sacc[mt][0] = sacc[mt][1] = pacc[mt][0] = pacc[mt][1] = zero4();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 aq = ld8(&Qs[(16 * mt + l16) * LDQ + 32 * ks + 8 * q4]);
        const bf16x8 ad = ld8(&dOs[(16 * mt + l16) * LDQ + 32 * ks + 8 * q4]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          sacc[mt][nt] = mfma16(aq, bk[nt][ks], sacc[mt][nt]);
          pacc[mt][nt] = mfma16(ad, bv[nt][ks], pacc[mt][nt]);
        }
      }

    // ---- P and dS (rows 16mt + 4q4 + e, key kw + 16nt + l16)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * mt + 4 * q4 + e;
        const float lr = lse_s[row], dr = dd_s[row];
        const int lim = tok_s[row] - blk * BLK;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int key = kw + 16 * nt + l16;
          const float p = key <= lim ? fast_exp2(sacc[mt][nt][e] * sl2 - lr) : 0.f;
          sacc[mt][nt][e] = p;
          pacc[mt][nt][e] = p * (pacc[mt][nt][e] - dr);
        }
      }

    // ---- dV += P^T dO, dK += dS^T Q  (owned keys along M, head dim along N, rows as K)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 ap[2], ad[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        ap[nt] = pack_ctiles(sacc[2 * ks][nt], sacc[2 * ks + 1][nt]);
        ad[nt] = pack_ctiles(pacc[2 * ks][nt], pacc[2 * ks + 1][nt]);
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const bf16x8 bdo = ld8(&dOsT[(16 * ct + l16) * LDT + 32 * ks + 8 * q4]);
        const bf16x8 bq = ld8(&QsT[(16 * ct + l16) * LDT + 32 * ks + 8 * q4]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          dva[nt][ct] = mfma16(ap[nt], bdo, dva[nt][ct]);
          dka[nt][ct] = mfma16(ad[nt], bq, dka[nt][ct]);
        }
      }
    }

    // ---- dS -> LDS as [row][key in kperm order]
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dSs[(16 * mt + 4 * q4 + e) * LDS_ + kw + kperm(16 * nt + l16)] = f2bf(pacc[mt][nt][e]);
    __syncthreads();

    // ---- dQ^T slice = K^T dS^T  (head dim along M, rows along N, all 128 keys as K)
    f32x4 dq[CW][4];
#pragma unroll
    for (int cw = 0; cw < CW; ++cw)
#pragma unroll
      for (int n2 = 0; n2 < 4; ++n2) dq[cw][n2] = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int n2 = 0; n2 < 4; ++n2) {
        const bf16x8 bds = ld8(&dSs[(16 * n2 + l16) * LDS_ + 32 * ks + 8 * q4]);
#pragma unroll
        for (int cw = 0; cw < CW; ++cw) dq[cw][n2] = mfma16(akt[cw][ks], bds, dq[cw][n2]);
      }
#pragma unroll
    for (int n2 = 0; n2 < 4; ++n2) {
      const int row = 16 * n2 + l16;
      const int p = pair_s[row];
      if (p < 0) continue;
      bf16raw* dst = dq_part + ((pair0 + (size_t)p) * R + row % R) * D + cbase + 4 * q4;
#pragma unroll
      for (int cw = 0; cw < CW; ++cw) {
        st4bf(dst + 16 * cw, dq[cw][n2][0] * scale, dq[cw][n2][1] * scale, dq[cw][n2][2] * scale,
              dq[cw][n2][3] * scale);
      }
    }
    __syncthreads();
  }

  // ---- dK, dV of the owned keys: lane holds head-dim column 16ct + l16, keys 4q4 + e
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const size_t rrow = (kv0 + (size_t)(kw + 16 * nt + 4 * q4 + e) * G) * D + l16;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        dk_acc[rrow + 16 * ct] += scale * dka[nt][ct][e];
        dv_acc[rrow + 16 * ct] += dva[nt][ct][e];
      }
    }
}

// D[row] = dot(dout[row], o[row]) over the head dim, fp32; D/8 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_dot(const bf16raw* __restrict__ o, const bf16raw* __restrict__ dout,
                                                 float* __restrict__ Dd, size_t rows) {
  constexpr int LPR = D / 8;
  const size_t row = (size_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  float s = 0.f;
  if (row < rows) {
    const uint4 a = *reinterpret_cast<const uint4*>(o + row * D + 8 * sub);
    const uint4 c = *reinterpret_cast<const uint4*>(dout + row * D + 8 * sub);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s += __uint_as_float(aw[i] << 16) * __uint_as_float(cw[i] << 16);
      s += __uint_as_float(aw[i] & 0xffff0000u) * __uint_as_float(cw[i] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (row < rows && sub == 0) Dd[row] = s;
}

// dq[b,t,g*R+hh,:] = sum of the token's valid per-slot partials (one wave per token/group).
template <int D, int R>
__global__ __launch_bounds__(256) void k_dq_combine(const int32_t* __restrict__ idx, const bf16raw* __restrict__ part,
                                                    bf16raw* __restrict__ dq, int T, int H, int G, int K, int t0,
                                                    int W, int rows) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int bg = row / W, tl = row % W, t = t0 + tl, b = bg / G, g = bg % G;
  const int32_t* ir = idx + ((size_t)bg * T + t) * K;
  const size_t p0 = (size_t)bg * W * K + (size_t)tl * K;
  const int last = t / BLK;
  constexpr int NCH = R * D / 4;
  for (int ch = lane; ch < NCH; ch += 64) {
    const int hh = ch / (D / 4), c4 = (ch % (D / 4)) * 4;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int s = 0; s < K; ++s) {
      const int bk = ir[s];
      if (bk < 0 || bk > last) continue;
      const uint2 raw = *reinterpret_cast<const uint2*>(part + ((p0 + s) * R + hh) * D + c4);
      a0 += __uint_as_float(raw.x << 16);
      a1 += __uint_as_float(raw.x & 0xffff0000u);
      a2 += __uint_as_float(raw.y << 16);
      a3 += __uint_as_float(raw.y & 0xffff0000u);
    }
    uint2 outw;
    outw.x = (uint32_t)f2bf(a0) | ((uint32_t)f2bf(a1) << 16);
    outw.y = (uint32_t)f2bf(a2) | ((uint32_t)f2bf(a3) << 16);
    *reinterpret_cast<uint2*>(dq + ((size_t)(b * T + t) * H + g * R + hh) * D + c4) = outw;
  }
}

__global__ __launch_bounds__(256) void k_fill_zero(float4* __restrict__ p, size_t n4) {
  for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

__global__ __launch_bounds__(256) void k_cvt_bf16(const float4* __restrict__ src, uint2* __restrict__ dst, size_t n4) {
  for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const float4 f = src[i];
    uint2 w;
    w.x = (uint32_t)f2bf(f.x) | ((uint32_t)f2bf(f.y) << 16);
    w.y = (uint32_t)f2bf(f.z) | ((uint32_t)f2bf(f.w) << 16);
    dst[i] = w;
  }
}

template <int D, int R>
static hipError_t bwd_partials_t(const Geo& g, const Win& w, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const uint16_t* dout, const float* lse, const float* Dd, const InvBufs& ib,
                                 uint16_t* dq_part, float* dk_acc, float* dv_acc, hipStream_t st) {
  dim3 grid(ib.max_items, g.B * g.G), block(256);
  k_bwd_kv<D, R><<<grid, block, 0, st>>>(q, k, v, dout, lse, Dd, ib.items, ib.item_count, ib.list, dq_part, dk_acc,
                                         dv_acc, g.T, g.H, g.G, g.K, w.t0, w.W, ib.max_items, g.scale,
                                         g.scale * LOG2E);
  return hipGetLastError();
}

template <int D, int R>
static hipError_t dq_combine_t(const Geo& g, const Win& w, const int32_t* idx, const uint16_t* dq_part, uint16_t* dq,
                               hipStream_t st) {
  const int rows = g.B * g.G * w.W;
  k_dq_combine<D, R><<<(rows + 3) / 4, 256, 0, st>>>(idx, dq_part, dq, g.T, g.H, g.G, g.K, w.t0, w.W, rows);
  return hipGetLastError();
}

#define MSA_DISPATCH_DR(FN, ...)                             \
  switch (g.D * 100 + g.R) {                                 \
    case 6401: return FN<64, 1>(__VA_ARGS__);                \
    case 6402: return FN<64, 2>(__VA_ARGS__);                \
    case 6404: return FN<64, 4>(__VA_ARGS__);                \
    case 6408: return FN<64, 8>(__VA_ARGS__);                \
    case 6416: return FN<64, 16>(__VA_ARGS__);               \
    case 12801: return FN<128, 1>(__VA_ARGS__);              \
    case 12802: return FN<128, 2>(__VA_ARGS__);              \
    case 12804: return FN<128, 4>(__VA_ARGS__);              \
    case 12808: return FN<128, 8>(__VA_ARGS__);              \
    case 12816: return FN<128, 16>(__VA_ARGS__);             \
    default: return hipErrorInvalidValue;                    \
  }

hipError_t launch_bwd_partials(const Geo& g, const Win& w, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const uint16_t* dout, const float* lse, const float* Dd, const InvBufs& ib,
                               uint16_t* dq_part, float* dk_acc, float* dv_acc, hipStream_t st) {
  MSA_DISPATCH_DR(bwd_partials_t, g, w, q, k, v, dout, lse, Dd, ib, dq_part, dk_acc, dv_acc, st)
}

hipError_t launch_dq_combine(const Geo& g, const Win& w, const int32_t* idx, const uint16_t* dq_part, uint16_t* dq,
                             hipStream_t st) {
  MSA_DISPATCH_DR(dq_combine_t, g, w, idx, dq_part, dq, st)
}

hipError_t launch_bwd_dot(const Geo& g, const uint16_t* o, const uint16_t* dout, float* Dd, hipStream_t st) {
  const size_t rows = (size_t)g.B * g.T * g.H;
  if (g.D == 128) {
    k_bwd_dot<128><<<(unsigned)((rows + 15) / 16), 256, 0, st>>>(o, dout, Dd, rows);
  } else if (g.D == 64) {
    k_bwd_dot<64><<<(unsigned)((rows + 31) / 32), 256, 0, st>>>(o, dout, Dd, rows);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t st) {
  const size_t n4 = n / 4;  // callers pass multiples of 4
  const unsigned grid = (unsigned)std::min<size_t>((n4 + 255) / 256, 8192);
  k_fill_zero<<<grid > 0 ? grid : 1, 256, 0, st>>>(reinterpret_cast<float4*>(p), n4);
  return hipGetLastError();
}

hipError_t launch_cvt_bf16(const float* src, uint16_t* dst, size_t n, hipStream_t st) {
  const size_t n4 = n / 4;
  const unsigned grid = (unsigned)std::min<size_t>((n4 + 255) / 256, 8192);
  k_cvt_bf16<<<grid > 0 ? grid : 1, 256, 0, st>>>(reinterpret_cast<const float4*>(src), reinterpret_cast<uint2*>(dst),
                                                   n4);
  return hipGetLastError();
}

}  // namespace msa
