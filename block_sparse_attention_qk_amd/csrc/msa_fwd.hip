// Main Branch forward for gfx950: exact softmax GQA attention over the cached
// blocks (ai-beat "flash-msa-sparse-attention-training", paragraph 1: the Main
// Branch runs exact softmax attention over only the selected blocks; xcelit
// "How MSA works": GQA main attention).
//
// KV-stationary schedule.  A work item is one (batch, group, block) and a run
// of the pairs that selected it.  Its K block (row-major) and V block
// (transposed) stay in LDS while tiles of 128 query rows (128/R tokens x R
// heads of the group) stream past.  For each pair the item writes the block's
// own softmax partial: o_b = sum_j e^{s_j - m_b} v_j / l_b (bf16) and
// lse_b = m_b + ln l_b (fp32).  A combine pass then forms the exact result
//   LSE = log sum_b e^{lse_b},  O = sum_b e^{lse_b - LSE} o_b.
// No atomics: every pair owns its partial slot.
#include "msa_common.h"
#include "msa_internal.h"

namespace msa {

template <int D, int R>
__global__ __launch_bounds__(256, 1) void k_fwd_kv(const bf16raw* __restrict__ q, const bf16raw* __restrict__ k,
                                                   const bf16raw* __restrict__ v, const int4* __restrict__ items,
                                                   const int32_t* __restrict__ item_count,
                                                   const int32_t* __restrict__ list, bf16raw* __restrict__ part_o,
                                                   float* __restrict__ part_lse, int T, int H, int G, int K,
                                                   int t0, int W, int max_items, float scale, float sl2) {
  constexpr int KS = D / 32;    // k-steps over the head dim
  constexpr int CT = D / 16;    // output column tiles
  constexpr int LDK = D + 8;    // K row stride (bf16)
  constexpr int LDV = BLK + 8;  // V^T row stride (bf16)
  constexpr int TT = 128 / R;   // tokens per 128-row tile
  __shared__ __attribute__((aligned(16))) bf16raw Ks[BLK * LDK];
  __shared__ __attribute__((aligned(16))) bf16raw Vt[D * LDV];

  const int bg = blockIdx.y;
  if ((int)blockIdx.x >= item_count[bg]) return;
  const int4 it = items[(size_t)bg * max_items + blockIdx.x];
  const int blk = it.x, start = it.y, len = it.z;
  const int b = bg / G, g = bg % G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, q4 = lane >> 4;
  const size_t kv0 = (size_t)(b * T + blk * BLK) * G + g;  // [B*T*G] row of key 0
  const size_t pair0 = (size_t)bg * W * K;
  const int32_t* lst = list + pair0 + start;

  for (int c = threadIdx.x; c < BLK * D / 8; c += 256) {
    const int r = c / (D / 8), c8 = c % (D / 8);
    st8(&Ks[r * LDK + 8 * c8], ld8(k + (kv0 + (size_t)r * G) * D + 8 * c8));
  }
  // V^T: two keys per 32-bit LDS word; keys of each 32-key step stored in kperm order.
  for (int u = threadIdx.x; u < 64 * (D / 8); u += 256) {
    const int kpl = u & 15, rest = u >> 4, cc = rest % (D / 8), grp = rest / (D / 8);
    const int key0 = 32 * grp + 2 * kpl;
    const uint4 v0 = ld16u(v + (kv0 + (size_t)key0 * G) * D + 8 * cc);
    const uint4 v1 = ld16u(v + (kv0 + (size_t)(key0 + 1) * G) * D + 8 * cc);
    const int pos = 32 * grp + kperm(2 * kpl);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t a = word_of(v0, m), c = word_of(v1, m);
      *reinterpret_cast<uint32_t*>(&Vt[(8 * cc + 2 * m) * LDV + pos]) = pair_lo(a, c);
      *reinterpret_cast<uint32_t*>(&Vt[(8 * cc + 2 * m + 1) * LDV + pos]) = pair_hi(a, c);
    }
  }
  __syncthreads();

  const int ntiles = (len + TT - 1) / TT;
  for (int tile = 0; tile < ntiles; ++tile) {
    int pr[2], tok[2], hh[2];
    bool val[2];
    bf16x8 bq[2][KS];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int row = 32 * wave + 16 * nt + l16;
      const int tt = row / R, li = tile * TT + tt;
      hh[nt] = row % R;
      val[nt] = li < len;
      pr[nt] = val[nt] ? lst[li] : 0;
      tok[nt] = t0 + pr[nt] / K;
      const bf16raw* qr = q + ((size_t)(b * T + tok[nt]) * H + g * R + hh[nt]) * D + 8 * q4;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bq[nt][ks] = val[nt] ? ld8(qr + 32 * ks) : zero8();
    }

    // S^T = K Q^T : keys along M (8 tiles), this wave's 32 rows along N (2 tiles)
    f32x4 acc[8][2];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[mt][0] = acc[mt][1] = zero4();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const bf16x8 a = ld8(&Ks[(16 * mt + l16) * LDK + 32 * ks + 8 * q4]);
        acc[mt][0] = mfma16(a, bq[0][ks], acc[mt][0]);
        acc[mt][1] = mfma16(a, bq[1][ks], acc[mt][1]);
      }

    float mrow[2], lrow[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int lim = val[nt] ? tok[nt] - blk * BLK : BLK - 1;  // keys past the query are masked
      float m = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float s = acc[mt][nt][e];
          if (16 * mt + 4 * q4 + e > lim) s = -INFINITY;
          acc[mt][nt][e] = s;
          m = fmaxf(m, s);
        }
      m = wave_max_xor_16_32(m);
      const float ms = m * sl2;
      float l = 0.f;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = fast_exp2(acc[mt][nt][e] * sl2 - ms);
          acc[mt][nt][e] = p;
          l += p;
        }
      mrow[nt] = m;
      lrow[nt] = wave_sum_xor_16_32(l);
    }

    // O^T = V^T P^T : head dim along M (CT tiles), rows along N, keys as K (4 steps)
    f32x4 oacc[CT][2];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) oacc[ct][0] = oacc[ct][1] = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 p0 = pack_ctiles(acc[2 * ks][0], acc[2 * ks + 1][0]);
      const bf16x8 p1 = pack_ctiles(acc[2 * ks][1], acc[2 * ks + 1][1]);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const bf16x8 a = ld8(&Vt[(16 * ct + l16) * LDV + 32 * ks + 8 * q4]);
        oacc[ct][0] = mfma16(a, p0, oacc[ct][0]);
        oacc[ct][1] = mfma16(a, p1, oacc[ct][1]);
      }
    }

#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      if (!val[nt]) continue;
      const float inv = 1.0f / lrow[nt];
      const size_t pidx = pair0 + (size_t)pr[nt];
      bf16raw* dst = part_o + (pidx * R + hh[nt]) * D + 4 * q4;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        st4bf(dst + 16 * ct, oacc[ct][nt][0] * inv, oacc[ct][nt][1] * inv, oacc[ct][nt][2] * inv,
              oacc[ct][nt][3] * inv);
      }
      if (q4 == 0) part_lse[pidx * R + hh[nt]] = mrow[nt] * scale + fast_log2(lrow[nt]) * LN2;
    }
  }
}

// One wavefront per (batch, group, token): exact log-sum-exp merge of the
// token's per-block partials.  A slot holds a partial iff its cache entry is a
// valid causal block.  A row with no valid entry gets O = 0, LSE = -inf.
template <int D, int R>
__global__ __launch_bounds__(256) void k_fwd_combine(const int32_t* __restrict__ idx, const bf16raw* __restrict__ part_o,
                                                     const float* __restrict__ part_lse, bf16raw* __restrict__ o,
                                                     float* __restrict__ lse, int T, int H, int G, int K, int t0,
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
    float M = -INFINITY;
    for (int s = 0; s < K; ++s) {
      const int bk = ir[s];
      if (bk >= 0 && bk <= last) M = fmaxf(M, part_lse[(p0 + s) * R + hh]);
    }
    float L = 0.f, a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    if (M != -INFINITY) {
      const float Ml = M * LOG2E;
      for (int s = 0; s < K; ++s) {
        const int bk = ir[s];
        if (bk < 0 || bk > last) continue;
        const float w = fast_exp2(part_lse[(p0 + s) * R + hh] * LOG2E - Ml);
        const uint2 raw = *reinterpret_cast<const uint2*>(part_o + ((p0 + s) * R + hh) * D + c4);
        L += w;
        a0 += w * __uint_as_float(raw.x << 16);
        a1 += w * __uint_as_float(raw.x & 0xffff0000u);
        a2 += w * __uint_as_float(raw.y << 16);
        a3 += w * __uint_as_float(raw.y & 0xffff0000u);
      }
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    const size_t orow = ((size_t)(b * T + t) * H + g * R + hh);
    uint2 outw;
    outw.x = (uint32_t)f2bf(a0 * inv) | ((uint32_t)f2bf(a1 * inv) << 16);
    outw.y = (uint32_t)f2bf(a2 * inv) | ((uint32_t)f2bf(a3 * inv) << 16);
    *reinterpret_cast<uint2*>(o + orow * D + c4) = outw;
    if (c4 == 0) lse[orow] = L > 0.f ? M + fast_log2(L) * LN2 : -INFINITY;
  }
}

template <int D, int R>
static hipError_t fwd_partials_t(const Geo& g, const Win& w, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const InvBufs& ib, uint16_t* part_o, float* part_lse, hipStream_t st) {
  dim3 grid(ib.max_items, g.B * g.G), block(256);
  k_fwd_kv<D, R><<<grid, block, 0, st>>>(q, k, v, ib.items, ib.item_count, ib.list, part_o, part_lse, g.T, g.H,
                                         g.G, g.K, w.t0, w.W, ib.max_items, g.scale, g.scale * LOG2E);
  return hipGetLastError();
}

template <int D, int R>
static hipError_t fwd_combine_t(const Geo& g, const Win& w, const int32_t* idx, const uint16_t* part_o,
                                const float* part_lse, uint16_t* o, float* lse, hipStream_t st) {
  const int rows = g.B * g.G * w.W;
  k_fwd_combine<D, R><<<(rows + 3) / 4, 256, 0, st>>>(idx, part_o, part_lse, o, lse, g.T, g.H, g.G, g.K, w.t0,
                                                       w.W, rows);
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

hipError_t launch_fwd_partials(const Geo& g, const Win& w, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const InvBufs& ib, uint16_t* part_o, float* part_lse, hipStream_t st) {
  MSA_DISPATCH_DR(fwd_partials_t, g, w, q, k, v, ib, part_o, part_lse, st)
}

hipError_t launch_fwd_combine(const Geo& g, const Win& w, const int32_t* idx, const uint16_t* part_o,
                              const float* part_lse, uint16_t* o, float* lse, hipStream_t st) {
  MSA_DISPATCH_DR(fwd_combine_t, g, w, idx, part_o, part_lse, o, lse, st)
}

}  // namespace msa
