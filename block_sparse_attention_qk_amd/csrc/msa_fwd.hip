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

#include <type_traits>

namespace msa {

// Position of 16-byte chunk c of row r in a swizzled row-major tile of DCH
// chunks per row (distinct LDS banks for 16-byte row reads and for transpose
// reads of 4 rows x 32 bytes).
template <int DCH>
__device__ __forceinline__ int fswz(int r, int c) {
  return c ^ ((((r & 3) << 2) | ((r >> 2) & 3)) & (DCH - 1));
}

// Each wave owns 32 query rows per tile (one MFMA column tile); the product is
// taken transposed, S^T = K Q^T with the 128 keys along M, so a lane holds 64
// keys of one row: the row max and sum are in-lane plus one cross-lane step.
// P^T then feeds O^T = V^T P^T as the B operand in place; V^T comes from the
// row-major V tile through LDS transpose reads.
template <int D, int R>
__global__ __launch_bounds__(256, 2) void k_fwd_kv(const bf16raw* __restrict__ q, const bf16raw* __restrict__ k,
                                                   const bf16raw* __restrict__ v, const int4* __restrict__ items,
                                                   const int32_t* __restrict__ item_count,
                                                   const int32_t* __restrict__ list, const int32_t* __restrict__ order,
                                                   bf16raw* __restrict__ part_o,
                                                   float* __restrict__ part_lse, int T, int H, int G, int K,
                                                   int t0, int W, int max_items, float scale, float sl2) {
  constexpr int KSD = D / 16;   // 32x32x16 k-steps over the head dim
  constexpr int NCT = D / 32;   // 32-wide head-dim tiles of O^T
  constexpr int DCH = D / 8;    // 16-byte chunks per row
  constexpr int TT = 128 / R;   // tokens per 128-row tile
  __shared__ __attribute__((aligned(16))) bf16raw Ks[BLK * D];
  __shared__ __attribute__((aligned(16))) bf16raw Vs[BLK * D];
  __shared__ int lsts[FWD_ITEM_TOKENS];  // the item's pair list (items hold at most FWD_ITEM_TOKENS pairs)

  // Groups run one after another in dispatch order (items are short, so the
  // order does not unbalance the launch): the Q rows the running items re-read
  // are one group's, a quarter of Q at G = 4, which stays in the last-level cache.
  // Within a group, items run in the order of their middle token (k_item_order).
  const int BG = (int)gridDim.x / max_items;
  const int bg = (int)blockIdx.x / max_items, slot = (int)blockIdx.x % max_items;
  if (slot >= item_count[bg]) return;
  const int item = order[(size_t)bg * max_items + slot];
  const int4 it = items[(size_t)bg * max_items + item];
  const int blk = it.x, start = it.y, len = it.z;
  const int b = bg / G, g = bg % G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5, g16 = lane >> 4, i16 = lane & 15;
  const size_t kv0 = (size_t)(b * T + blk * BLK) * G + g;
  const size_t pair0 = (size_t)bg * W * K;
  const int32_t* lst = list + pair0 + start;

  {
    constexpr int NLD = BLK * DCH / 256;  // 16-byte chunks per thread and matrix
    uint4 kr[NLD], vr[NLD];
#pragma unroll
    for (int u = 0; u < NLD; ++u) {  // all loads first, then all LDS stores
      const int c = tid + 256 * u, r = c / DCH, cc = c % DCH;
      const size_t src = (kv0 + (size_t)r * G) * D + 8 * cc;
      kr[u] = ld16u(k + src);
      vr[u] = ld16u(v + src);
    }
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int c = tid + 256 * u, r = c / DCH, cc = c % DCH;
      st16u(&Ks[r * D + 8 * fswz<DCH>(r, cc)], kr[u]);
      st16u(&Vs[r * D + 8 * fswz<DCH>(r, cc)], vr[u]);
    }
    for (int i = tid; i < len; i += 256) lsts[i] = lst[i];
  }

  // this lane's query row within a tile and its Q operand (B of S^T: column = row).
  // Loads never branch: a row past the list reads the list's last entry
  // (finite data; its result is dropped).  The list entries come from LDS, so
  // the only global loads in the loop are the Q rows: waiting for them never
  // waits for the partial stores issued after them.
  const int row = 32 * wave + l32;
  const int tt = row / R, hh = row % R;
  auto list_entry = [&](int ti) { return lsts[min(ti * TT + tt, len - 1)]; };
  auto load_q = [&](int ti, int ent, bf16x8* bq, int& pr, int& lim) {
    const bool val = ti * TT + tt < len;
    const int tl = ent >> LIST_SLOT_BITS, t = t0 + tl;
    pr = val ? tl * K + (ent & ((1 << LIST_SLOT_BITS) - 1)) : -1;
    lim = val ? t - blk * BLK : BLK - 1;
    const bf16raw* qr = q + ((size_t)(b * T + t) * H + g * R + hh) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) bq[ks] = ld8(qr + 16 * ks);
  };

  const int ntiles = (len + TT - 1) / TT;
  bf16x8 bq[KSD];
  int pr = -1, lim = BLK - 1;
  if (ntiles > 0) load_q(0, lst[min(tt, len - 1)], bq, pr, lim);
  // The prologue's loads complete here and the first Q operand is redefined
  // by a non-memory op, so that the loop's waits count only its own traffic.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
#pragma unroll
  for (int ks = 0; ks < KSD; ++ks) asm volatile("" : "+v"(bq[ks]));
  __syncthreads();

  // Only a block's first item can hold the block's own tokens, whose rows
  // need the causal mask inside the block; every other item runs the loop
  // without the per-key compares.
  auto tiles = [&](auto maskc) {
  constexpr bool MASK = decltype(maskc)::value;
  for (int ti = 0; ti < ntiles; ++ti) {
    const int pair1 = list_entry(ti + 1);
    // S^T = K Q^T: 4 key tiles of 32 along M, this wave's 32 rows along N
    f32x16 acc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) acc[kt] = zero16();
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int kr = 32 * kt + l32;
        acc[kt] = mfma32(ld8(&Ks[kr * D + 8 * fswz<DCH>(kr, 2 * ks + h)]), bq[ks], acc[kt]);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the K operand loads of later steps from piling up in registers
    }
    const int cpr = pr, clim = lim;

    // softmax over the block's keys of this row: lane holds keys 32kt + 8j + 4h + i
    float m = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int kk = 32 * kt + 8 * (e >> 2) + 4 * h + (e & 3);
        const float sv = MASK && kk > clim ? -INFINITY : acc[kt][e];
        acc[kt][e] = sv;
        m = fmaxf(m, sv);
      }
    m = fmaxf(m, __shfl_xor(m, 32));
    const float ms = m * sl2;
    float l = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pv = fast_exp2(acc[kt][e] * sl2 - ms);
        acc[kt][e] = pv;
        l += pv;
      }
    l += __shfl_xor(l, 32);

    // P^T as bf16 B operands (K step s = keys of tile s/2, C elements 8(s%2)..+7)
    bf16x8 bp[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int kt = s >> 1, ss = s & 1;
      bp[s] = as_bf8(make_uint4(
          pack2(acc[kt][8 * ss + 0], acc[kt][8 * ss + 1]), pack2(acc[kt][8 * ss + 2], acc[kt][8 * ss + 3]),
          pack2(acc[kt][8 * ss + 4], acc[kt][8 * ss + 5]), pack2(acc[kt][8 * ss + 6], acc[kt][8 * ss + 7])));
    }

    load_q(ti + 1, pair1, bq, pr, lim);  // next tile's rows in flight during PV (past the end: unused)

    // O^T = V^T P^T: head dim along M (NCT tiles), rows along N, keys as K (8 steps of 16)
    f32x16 oacc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) oacc[ct] = zero16();
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int kt = s >> 1, ss = s & 1;
      const int kr = 32 * kt + 16 * ss + 4 * h + (i16 >> 2);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int col = 32 * ct + 16 * (g16 & 1) + 4 * (i16 & 3);
        const uint2 a0 = lds_tr4(&Vs[kr * D + 8 * fswz<DCH>(kr, col >> 3) + (col & 7)]);
        const uint2 a1 = lds_tr4(&Vs[(kr + 8) * D + 8 * fswz<DCH>(kr + 8, col >> 3) + (col & 7)]);
        oacc[ct] = mfma32(as_bf8(make_uint4(a0.x, a0.y, a1.x, a1.y)), bp[s], oacc[ct]);
      }
    }

    // lane holds row `row`, head-dim columns 32ct + 8j + 4h + (0..3)
    // Stores never branch (so the next tile's loads are waited on alone): a
    // row past the list writes the spare slot after the window's pairs.
    {
      const float inv = 1.0f / l;
      const size_t pidx = cpr >= 0 ? pair0 + (size_t)cpr : (size_t)BG * W * K;
      // Lane halves h = 0/1 hold head-dim columns 8j + 0..3 / 8j + 4..7 of the
      // same row; one lane swap per dword gives lane h whole 16-byte runs
      // (run 2k + h, k = 2ct + pp, = columns 16k + 8h .. +7), stored as one
      // 16-byte write into the pair's slot in the run-interleaved layout, where
      // one store instruction fills 256 contiguous bytes of each of its pairs.
      bf16raw* dst = part_o + pidx * R * D + 16 * hh + 8 * h;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const int e0 = 8 * pp, e1 = 8 * pp + 4;  // columns 16pp + 4h + 0..3 and 16pp + 8 + 4h + 0..3
          const uint32_t u0 = pack2(oacc[ct][e0] * inv, oacc[ct][e0 + 1] * inv);
          const uint32_t u1 = pack2(oacc[ct][e0 + 2] * inv, oacc[ct][e0 + 3] * inv);
          const uint32_t w0 = pack2(oacc[ct][e1] * inv, oacc[ct][e1 + 1] * inv);
          const uint32_t w1 = pack2(oacc[ct][e1 + 2] * inv, oacc[ct][e1 + 3] * inv);
          const auto s0 = __builtin_amdgcn_permlane32_swap(u0, w0, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(u1, w1, false, false);
          st16nt(dst + 16 * R * (2 * ct + pp), make_uint4(s0[0], s1[0], s0[1], s1[1]));
        }
      part_lse[pidx * R + hh] = m * scale + fast_log2(l) * LN2;  // both lane halves hold the same value
    }
  }
  };
  if (it.w & ITEM_DIAG)
    tiles(std::true_type{});
  else
    tiles(std::false_type{});
}

// Exact log-sum-exp merge of a token's per-block partials, one (batch,
// group, token) row per R*D/8 threads (each thread owns 8 head-dim values of
// one head and streams 16 bytes per slot).  A slot holds a partial iff its
// cache entry is a valid causal block.  A row with no valid entry gets
// O = 0, LSE = -inf; a row with a NaN partial (NaN inputs) gets NaN.  WITH_D (the merged forward/backward call) also forms the
// backward's D = rowsum(dout * O) here, while O is still in registers.
template <int D, int R, bool WITH_D>
__global__ __launch_bounds__(256) void k_fwd_combine(const int32_t* __restrict__ idx, const bf16raw* __restrict__ part_o,
                                                     const float* __restrict__ part_lse, bf16raw* __restrict__ o,
                                                     float* __restrict__ lse, const bf16raw* __restrict__ dout,
                                                     float* __restrict__ Dd, int T, int H, int G, int K, int t0,
                                                     int W, int rows) {
  constexpr int TPR = R * D / 8;  // threads per row
  constexpr int RPB = 256 / TPR;  // rows per block
  const int sub = threadIdx.x % TPR;
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= rows) return;
  const int bg = row / W, tl = row % W, t = t0 + tl, b = bg / G, g = bg % G;
  const int hh = sub / (D / 8), run = sub % (D / 8), c8 = run * 8;
  const int32_t* ir = idx + ((size_t)bg * T + t) * K;
  const size_t p0 = (size_t)bg * W * K + (size_t)tl * K;
  const unsigned last = (unsigned)(t / BLK);
  const float* pl = part_lse + p0 * R + hh;
  const bf16raw* po = part_o + p0 * R * D + partial_run_offset<R>(hh, run);
  const size_t orow = (size_t)(b * T + t) * H + g * R + hh;
  uint4 dch = make_uint4(0u, 0u, 0u, 0u);
  if constexpr (WITH_D) dch = ld16u(dout + orow * D + c8);  // issued ahead of the slot stream

  // One pass with a running maximum: each batch loads its slots' cache
  // entries, lse and partial rows together (slots past K re-read the last one;
  // a slot without a partial is read and then masked, so no load waits on a
  // branch), and the accumulator is rescaled when the maximum grows.
  constexpr int SB = 16;  // slots per batch: independent loads in flight per thread
  float M = -INFINITY, L = 0.f, acc[8];
  bool nan_seen = false;  // a NaN partial lse (the running max would skip it) makes the row NaN
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int s0 = 0; s0 < K; s0 += SB) {
    int ent[SB];
    float lv[SB];
    uint4 raw[SB];
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int s = min(s0 + u, K - 1);
      ent[u] = ir[s];
      lv[u] = pl[(size_t)s * R];
      raw[u] = ld16nt(po + (size_t)s * R * D);
    }
    // keep every load above the masking (the compiler would otherwise sink one
    // into a branch and issue it after the rest, costing a second round trip)
#pragma unroll
    for (int u = 0; u < SB; ++u) asm volatile("" : "+v"(raw[u].x), "+v"(raw[u].y), "+v"(raw[u].z), "+v"(raw[u].w));
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const bool ok = s0 + u < K && (unsigned)ent[u] <= last;
      lv[u] = ok ? lv[u] : -INFINITY;
      raw[u] = ok ? raw[u] : make_uint4(0u, 0u, 0u, 0u);
    }
    float mb = M;
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      mb = fmaxf(mb, lv[u]);
      nan_seen |= lv[u] != lv[u];
    }
    if (mb == -INFINITY) continue;  // no valid slot yet
    const float mbl = mb * LOG2E;
    const float c = fast_exp2(M * LOG2E - mbl);  // 0 while M is still -inf
    L *= c;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= c;
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const float w = fast_exp2(lv[u] * LOG2E - mbl);  // 0 for an invalid slot
      L += w;
      const uint32_t wd[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        acc[2 * m] += w * __uint_as_float(wd[m] << 16);
        acc[2 * m + 1] += w * __uint_as_float(wd[m] & 0xffff0000u);
      }
    }
    M = mb;
  }
  const float inv = nan_seen ? __builtin_nanf("") : L > 0.f ? 1.0f / L : 0.f;
  const uint4 ob = make_uint4(pack2(acc[0] * inv, acc[1] * inv), pack2(acc[2] * inv, acc[3] * inv),
                              pack2(acc[4] * inv, acc[5] * inv), pack2(acc[6] * inv, acc[7] * inv));
  st16u(o + orow * D + c8, ob);
  if (c8 == 0) lse[orow] = nan_seen ? __builtin_nanf("") : L > 0.f ? M + fast_log2(L) * LN2 : -INFINITY;
  if constexpr (WITH_D) {
    // D = rowsum(dout * o) of the bf16 o just written, summed in the order of
    // k_bwd_dot (8 products per lane, then xor shuffles over the D/8 lanes of
    // the head), so the merged call reproduces msa_bwd's D bit for bit.
    const uint32_t aw[4] = {ob.x, ob.y, ob.z, ob.w}, cw[4] = {dch.x, dch.y, dch.z, dch.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s += __uint_as_float(aw[i] << 16) * __uint_as_float(cw[i] << 16);
      s += __uint_as_float(aw[i] & 0xffff0000u) * __uint_as_float(cw[i] & 0xffff0000u);
    }
#pragma unroll
    for (int off = D / 16; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (c8 == 0) Dd[orow] = s;
  }
}

template <int D, int R>
static hipError_t fwd_partials_t(const Geo& g, const Win& w, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const InvBufs& ib, uint16_t* part_o, float* part_lse, hipStream_t st) {
  if ((long long)ib.max_items * g.B * g.G > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  dim3 grid(ib.max_items * g.B * g.G), block(256);
  // Items in the order of their middle token: the running items then gather
  // query rows from a narrow token range, which the L2 and the last-level cache
  // serve far better than rows spread over the whole window.
  if (const hipError_t e = launch_item_order(g, w, ib, st); e != hipSuccess) return e;
  k_fwd_kv<D, R><<<grid, block, 0, st>>>(q, k, v, ib.items, ib.item_count, ib.list, ib.order, part_o, part_lse, g.T,
                                         g.H, g.G, g.K, w.t0, w.W, ib.max_items, g.scale, g.scale * LOG2E);
  return hipGetLastError();
}

template <int D, int R>
static hipError_t fwd_combine_t(const Geo& g, const Win& w, const int32_t* idx, const uint16_t* part_o,
                                const float* part_lse, uint16_t* o, float* lse, const uint16_t* dout, float* Dd,
                                hipStream_t st) {
  const int rows = g.B * g.G * w.W;
  constexpr int RPB = 256 / (R * D / 8);
  if (dout != nullptr)
    k_fwd_combine<D, R, true><<<(rows + RPB - 1) / RPB, 256, 0, st>>>(idx, part_o, part_lse, o, lse, dout, Dd, g.T,
                                                                      g.H, g.G, g.K, w.t0, w.W, rows);
  else
    k_fwd_combine<D, R, false><<<(rows + RPB - 1) / RPB, 256, 0, st>>>(idx, part_o, part_lse, o, lse, nullptr,
                                                                       nullptr, g.T, g.H, g.G, g.K, w.t0, w.W, rows);
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
                              const float* part_lse, uint16_t* o, float* lse, const uint16_t* dout, float* Dd,
                              hipStream_t st) {
  MSA_DISPATCH_DR(fwd_combine_t, g, w, idx, part_o, part_lse, o, lse, dout, Dd, st)
}

}  // namespace msa
