// Main Branch backward for gfx950: dQ, dK, dV of exact softmax GQA attention
// over the cached blocks (ai-beat "flash-msa-sparse-attention-training",
// paragraph 2: training needs a backward pass through the sparse pattern;
// keyed on the cached block indices, xcelit "How MSA works").
//
// KV-stationary schedule, one work item per (batch, group, block) and window.
// Eight waves share one 128-key block in two roles, one wave of each role per
// SIMD, so that every SIMD always has a VALU-heavy and an MFMA-heavy wave:
//   producers (waves 0-3), key quarter kq: for query tile i+1,
//     S = Q K^T and dP = dO V^T (32 rows x its 32 keys; K, V rows in registers),
//     P = exp(scale S - LSE) (zero past the query), dS = scale P (dP - D),
//     P^T and dS^T -> LDS; and they gather the query rows of tile i+3.
//   consumers (waves 4-7), cw = wave - 4: for tile i,
//     dV += P^T dO, dK += dS^T Q   (key half cw/2 x head-dim half cw%2),
//     dQ^T = K^T dS^T               (head-dim tile cw x the 32 rows),
//   one barrier per tile.  Query tiles (32 rows = 32/R tokens x R heads) are
// triple-buffered in LDS, P^T/dS^T double-buffered; every LDS tile is
// XOR-swizzled on 16-byte chunks (v_mfma_f32_32x32x16_bf16 operands by 16-byte
// reads and by ds_read_b64_tr_b16 transpose reads).
// Items are dispatched in the order of the middle token of their run.
// dQ leaves as one bf16 partial per (token, slot); a combine pass sums a
// token's partials.  dK/dV are added into fp32 accumulators once per item
// (atomically only when a block's list is cut into several items).
#include "msa_common.h"
#include "msa_internal.h"

#include <algorithm>
#include <type_traits>

namespace msa {

// Position of 16-byte chunk c of row r in a swizzled row-major tile of
// DCH chunks per row: consecutive rows land on distinct LDS banks both for
// 16-byte row reads and for transpose reads of 4 rows x 32 bytes.
template <int DCH>
__device__ __forceinline__ int swz(int r, int c) {
  return c ^ ((((r & 3) << 2) | ((r >> 2) & 3)) & (DCH - 1));
}

// Position of 16-byte chunk c of key row r in a P^T / dS^T tile (32 query rows
// = 4 chunks per key row, four key rows per 256-byte bank line): the 8-byte
// writes after the softmax, the 16-byte operand reads of dV/dK and the
// transpose reads of dQ each spread evenly over the banks.
__device__ __forceinline__ int pswz(int r, int c) { return c ^ ((r >> 2) & 3); }

constexpr int BWD_THREADS = 512;
constexpr int BWD_TR = 32;  // query rows per tile

template <int D, int R>
__global__ __launch_bounds__(BWD_THREADS, 2) void k_bwd_kv(
    const bf16raw* __restrict__ q, const bf16raw* __restrict__ k, const bf16raw* __restrict__ v,
    const bf16raw* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dd,
    const int4* __restrict__ items, const int32_t* __restrict__ item_count, const int32_t* __restrict__ list,
    const int32_t* __restrict__ order, bf16raw* __restrict__ dq_part, float* __restrict__ dk_acc,
    float* __restrict__ dv_acc, int T, int H, int G, int K, int t0, int W, int max_items, float scale, float sl2) {
  constexpr int KSD = D / 16;    // 32x32x16 k-steps over the head dim
  constexpr int NCT = D / 32;    // 32-wide head-dim tiles
  constexpr int DCH = D / 8;     // 16-byte chunks per row
  constexpr int TR = BWD_TR;     // query rows per tile
  constexpr int TT = TR / R;     // tokens per tile
  constexpr int CPT = DCH / 8;   // staged chunks per producer thread and matrix (8 threads per row)
  __shared__ __attribute__((aligned(16))) bf16raw Ks[BLK * D];
  __shared__ __attribute__((aligned(16))) bf16raw Qs[3][TR * D];
  __shared__ __attribute__((aligned(16))) bf16raw dOs[3][TR * D];
  __shared__ __attribute__((aligned(16))) bf16raw PT[2][BLK * TR];
  __shared__ __attribute__((aligned(16))) bf16raw dST[2][BLK * TR];
  __shared__ __attribute__((aligned(16))) float rlse[3][TR];
  __shared__ __attribute__((aligned(16))) float rdd[3][TR];
  __shared__ __attribute__((aligned(16))) int rlim[3][TR];
  __shared__ __attribute__((aligned(16))) int rpair[3][TR];
  __shared__ int lsts[BWD_ITEM_TOKENS];  // the item's pair list

  // Groups run one after another in dispatch order, and a group's items in
  // the order of their middle token (k_item_order): the query and dO rows that
  // the running items gather then come from one group and a narrow token
  // range, which the last-level cache holds far better than all of a group's
  // rows (items are capped at BWD_ITEM_TOKENS pairs, so no single item
  // dominates the tail).
  const int bg = (int)blockIdx.x / max_items, slot = (int)blockIdx.x % max_items;
  if (slot >= item_count[bg]) return;
  const int item = order[(size_t)bg * max_items + slot];
  const int4 it = items[(size_t)bg * max_items + item];
  const int blk = it.x, start = it.y, len = it.z;
  const int b = bg / G, g = bg % G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5, g16 = (lane >> 4) & 1, i16 = lane & 15;
  const int kq = wave & 3;
  const size_t kv0 = (size_t)(b * T + blk * BLK) * G + g;
  const size_t pair0 = (size_t)bg * W * K;
  const int32_t* lst = list + pair0 + start;
  const int kown = 32 * kq + l32;  // this lane's key
  const int ntiles = (len + TT - 1) / TT;

  // ---- K block -> LDS (swizzled row-major), all threads: loads first, then stores
  {
    constexpr int NLD = BLK * DCH / BWD_THREADS;
    uint4 kr[NLD];
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int c = tid + BWD_THREADS * u;
      kr[u] = ld16u(k + (kv0 + (size_t)(c / DCH) * G) * D + 8 * (c % DCH));
    }
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int c = tid + BWD_THREADS * u, r = c / DCH, cc = c % DCH;
      st16u(&Ks[r * D + 8 * swz<DCH>(r, cc)], kr[u]);
    }
    // The pair list goes to LDS, so that the producer's only global loads in
    // its loop are the staged rows (a list lookup would otherwise wait for the
    // staging loads issued before it).
    for (int i = tid; i < len; i += BWD_THREADS) lsts[i] = lst[i];
  }
  __syncthreads();

  if (wave < 4) {
    // =================== producer ===================
    // own-key K and V rows as B operands of S and dP (key kown, head dims 16ks + 8h .. +7)
    bf16x8 bk[KSD], bv[KSD];
    {
      const bf16raw* kr = k + (kv0 + (size_t)kown * G) * D + 8 * h;
      const bf16raw* vr = v + (kv0 + (size_t)kown * G) * D + 8 * h;
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        bk[ks] = ld8(kr + 16 * ks);
        bv[ks] = ld8(vr + 16 * ks);
      }
    }
    // Staging: producer thread tid owns tile row tid/8 and chunks (tid%8) + 8u.
    // A tile's rows are loaded two iterations before they go to LDS, into one
    // of two register sets (tile parity), so each load has two tile times to
    // arrive.  Loads never branch and never wait where they are issued: a row
    // past the list reads the list's last entry (finite data, masked at store
    // time), list entries come from LDS, and scaling and validity are applied
    // when the staged registers go to LDS.
    // Operand offsets of this lane: row l32's chunk 2ks + h is xq0 ^ 16ks
    // (the swizzle is an XOR on the chunk bits), and key kown's P^T/dS^T run
    // jj is xw0 ^ 8jj; the bases are made opaque per tile so that the eight
    // offsets are formed next to their reads, not held in registers.
    const int xq0 = l32 * D + 8 * swz<DCH>(l32, h), xw0 = kown * TR + 8 * pswz(kown, 0) + 4 * h;
    const int srow = tid >> 3, ssub = tid & 7;
    uint4 sq[2][CPT], sdo[2][CPT];
    int s_li[2] = {len, len}, s_ent[2] = {0, 0};
    float s_lse[2] = {0.f, 0.f}, s_dd[2] = {0.f, 0.f};
    auto list_entry = [&](int ti) { return lsts[min(ti * TT + srow / R, len - 1)]; };
    auto stage_load = [&](auto setc, int ti, int ent) {
      constexpr int st = decltype(setc)::value;
      s_li[st] = ti * TT + srow / R;
      s_ent[st] = ent;
      const int t = t0 + (ent >> LIST_SLOT_BITS);
      const size_t hrow = (size_t)(b * T + t) * H + g * R + srow % R;
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        sq[st][u] = ld16u(q + hrow * D + 8 * (ssub + 8 * u));
        sdo[st][u] = ld16u(dout + hrow * D + 8 * (ssub + 8 * u));
      }
      s_lse[st] = lse[hrow];
      s_dd[st] = Dd[hrow];
    };
    auto stage_store = [&](auto setc, int buf) {
      constexpr int st = decltype(setc)::value;
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int off = srow * D + 8 * swz<DCH>(srow, ssub + 8 * u);
        st16u(&Qs[buf][off], sq[st][u]);
        st16u(&dOs[buf][off], sdo[st][u]);
      }
      // The row's 8 threads hold the same values and all write them: no branch,
      // so the waits for the staging loads stay exact.
      const bool val = s_li[st] < len;  // a row past the list: P = 0 (LSE = +inf), no key allowed, no dQ
      const int tl = s_ent[st] >> LIST_SLOT_BITS;
      rlse[buf][srow] = val ? s_lse[st] * LOG2E : INFINITY;
      rdd[buf][srow] = s_dd[st] * scale;
      rlim[buf][srow] = val ? t0 + tl - blk * BLK : -1;
      rpair[buf][srow] = val ? tl * K + (s_ent[st] & ((1 << LIST_SLOT_BITS) - 1)) : -1;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;

    stage_load(I0{}, 0, list_entry(0));
    stage_store(I0{}, 0);
    // All prologue loads (K and V operands included) complete here, so that the
    // loop's waits count only its own traffic.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) asm volatile("" : "+v"(bk[ks]), "+v"(bv[ks]));
    stage_load(I1{}, 1, list_entry(1));
    stage_load(I0{}, 2, list_entry(2));
    // Drained once per item: the loop is then entered with no load in flight,
    // so the compiler's waits inside it count only the loop's own staging
    // loads (a load pending from here would make it wait for all of them at
    // the loop head, once per six tiles).
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    __syncthreads();

    // One iteration: compute tile i+1, stage tile i+2, load tile i+4.  The
    // buffer and register-set indices are compile-time constants in each copy
    // of the 6-way unrolled loop ((i+1) mod 3, (i+1) mod 2, (i+2) mod 3 and
    // i mod 2, the set that tile i+2 arrived in and tile i+4 loads into).
    // MASK: only a block's first item can hold the block's own tokens, whose
    // keys past the query are masked; other items skip the per-key compares.
    auto produce = [&](auto maskc, auto qbc, auto pbc, auto sbc, auto setc, int i) {
      constexpr bool MASK = decltype(maskc)::value;
      constexpr int qb = decltype(qbc)::value, pb = decltype(pbc)::value, sb = decltype(sbc)::value;
      const int pair4 = list_entry(i + 4);  // for this iteration's staging load
      if (i + 1 < ntiles) {
        const bf16raw* Qc = Qs[qb];
        const bf16raw* dOc = dOs[qb];
        int xq = xq0, xw = xw0;
        asm volatile("" : "+v"(xq), "+v"(xw));
        f32x16 sacc = zero16(), pacc = zero16();
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          const int off = xq ^ (16 * ks);
          sacc = mfma32(ld8(&Qc[off]), bk[ks], sacc);
          pacc = mfma32(ld8(&dOc[off]), bv[ks], pacc);
        }
        // lane holds key kown and rows 8jj + 4h + ii
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r0 = 8 * jj + 4 * h;
          const float4 lv = *reinterpret_cast<const float4*>(&rlse[qb][r0]);
          const float4 dv4 = *reinterpret_cast<const float4*>(&rdd[qb][r0]);
          const float la[4] = {lv.x, lv.y, lv.z, lv.w}, da[4] = {dv4.x, dv4.y, dv4.z, dv4.w};
          int ma[4] = {BLK, BLK, BLK, BLK};
          if constexpr (MASK) {
            const int4 lm = *reinterpret_cast<const int4*>(&rlim[qb][r0]);
            ma[0] = lm.x;
            ma[1] = lm.y;
            ma[2] = lm.z;
            ma[3] = lm.w;
          }
          float pv[4], dsv[4];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int e = 4 * jj + ii;
            const float ex = fast_exp2(sacc[e] * sl2 - la[ii]);
            pv[ii] = !MASK || kown <= ma[ii] ? ex : 0.f;
            dsv[ii] = pv[ii] * fmaf(pacc[e], scale, -da[ii]);
          }
          const int o = xw ^ (8 * jj);
          *reinterpret_cast<uint2*>(&PT[pb][o]) = make_uint2(pack2(pv[0], pv[1]), pack2(pv[2], pv[3]));
          *reinterpret_cast<uint2*>(&dST[pb][o]) = make_uint2(pack2(dsv[0], dsv[1]), pack2(dsv[2], dsv[3]));
        }
      }
      stage_store(setc, sb);  // tile i+2 (rows past the list are masked)
      stage_load(setc, i + 4, pair4);
      __syncthreads();
    };
    // i0 = -1 (mod 6): i0 + u computes tile 6m + u; the register set is (i0 + u) mod 2 = (u + 1) mod 2.
    // The six steps run unconditionally (steps past the last tile only stage
    // clamped rows), so the loop body is straight-line code and the waits for
    // the staging loads count exactly; the consumer runs the same steps.
    auto loop = [&](auto mc) {
      for (int i0 = -1; i0 < ntiles; i0 += 6) {
        produce(mc, I0{}, I0{}, I1{}, I1{}, i0);
        produce(mc, I1{}, I1{}, I2{}, I0{}, i0 + 1);
        produce(mc, I2{}, I0{}, I0{}, I1{}, i0 + 2);
        produce(mc, I0{}, I1{}, I1{}, I0{}, i0 + 3);
        produce(mc, I1{}, I0{}, I2{}, I1{}, i0 + 4);
        produce(mc, I2{}, I1{}, I0{}, I0{}, i0 + 5);
      }
    };
    // Each loop drains its loads at its exit (two different wait forms, so that
    // the two are not merged into one shared exit block): the loops share exit
    // and entry checks, and a load of the masked loop still in flight on that
    // path would make the compiler wait early inside the unmasked loop.
    if (it.w & ITEM_DIAG) {
      loop(std::true_type{});
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    } else {
      loop(std::false_type{});
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    }
  } else {
    // =================== consumer ===================
    // Consumer cw = wave - 4 owns keys 64kh .. 64kh+63 (two 32-key tiles kt)
    // and head-dim tiles NCC dh .. NCC dh + NCC - 1 of dV and dK: each P^T/dS^T
    // operand read feeds NCC MFMAs (its dim tiles) and each dO/Q operand read
    // two (both key tiles).
    constexpr int NCC = NCT / 2;  // head-dim tiles per consumer
    const int cw = wave - 4, kh = cw >> 1, dh = cw & 1;
    f32x16 dka[2][NCC], dva[2][NCC];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int cc = 0; cc < NCC; ++cc) dka[kt][cc] = dva[kt][cc] = zero16();
    __syncthreads();  // K block and tile 0 staged

    // One tile: the buffer indices are compile-time constants in each copy of
    // the 6-way unrolled loop (i mod 3 and i mod 2), so every LDS address is a
    // lane offset plus an immediate.
    auto consume = [&](auto qbc, auto pbc, int i) {
      constexpr int qb = decltype(qbc)::value, pb = decltype(pbc)::value;
      if (i >= 0 && i < ntiles) {
        const bf16raw* Qc = Qs[qb];
        const bf16raw* dOc = dOs[qb];
        // ---- dV += P^T dO, dK += dS^T Q : own 64 keys x own 64 head dims, the tile's 32 rows
#pragma unroll
        for (int st = 0; st < TR / 16; ++st) {
          bf16x8 ap[2], ad[2];
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            const int key = 64 * kh + 32 * kt + l32;
            ap[kt] = ld8(&PT[pb][key * TR + 8 * pswz(key, 2 * st + h)]);
            ad[kt] = ld8(&dST[pb][key * TR + 8 * pswz(key, 2 * st + h)]);
          }
          const int ra = 16 * st + 8 * h + (i16 >> 2);  // rows of the first transpose read
#pragma unroll
          for (int cc = 0; cc < NCC; ++cc) {
            const int col = 32 * (NCC * dh + cc) + 16 * g16 + 4 * (i16 & 3);
            const int oa = ra * D + 8 * swz<DCH>(ra, col >> 3) + (col & 7);
            const int ob = (ra + 4) * D + 8 * swz<DCH>(ra + 4, col >> 3) + (col & 7);
            const uint2 d0 = lds_tr4(&dOc[oa]), d1 = lds_tr4(&dOc[ob]);
            const uint2 q0 = lds_tr4(&Qc[oa]), q1 = lds_tr4(&Qc[ob]);
            const bf16x8 bd = as_bf8(make_uint4(d0.x, d0.y, d1.x, d1.y));
            const bf16x8 bq = as_bf8(make_uint4(q0.x, q0.y, q1.x, q1.y));
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
              dva[kt][cc] = mfma32(ap[kt], bd, dva[kt][cc]);
              dka[kt][cc] = mfma32(ad[kt], bq, dka[kt][cc]);
            }
          }
        }
        // ---- dQ^T tile = K^T dS^T : head-dim tile kq along M, the 32 rows along N, keys as K
        if (kq < NCT) {
          // Both swizzles depend only on bits 0..3 of the row, which a step of 16
          // keys leaves unchanged: k-step ks reads at a per-lane base plus a
          // constant (16 rows of Ks, 16 rows of dS^T), and its operands are
          // read two steps ahead of its MFMA.
          const int kr0 = 8 * h + (i16 >> 2);
          const int col = 32 * kq + 16 * g16 + 4 * (i16 & 3);
          const int rc = 16 * g16 + 4 * (i16 & 3);
          const bf16raw* ka0 = &Ks[kr0 * D + 8 * swz<DCH>(kr0, col >> 3) + (col & 7)];
          const bf16raw* ka1 = &Ks[(kr0 + 4) * D + 8 * swz<DCH>(kr0 + 4, col >> 3) + (col & 7)];
          const bf16raw* db0 = &dST[pb][kr0 * TR + 8 * pswz(kr0, rc >> 3) + (rc & 7)];
          const bf16raw* db1 = &dST[pb][(kr0 + 4) * TR + 8 * pswz(kr0 + 4, rc >> 3) + (rc & 7)];
          uint2 qa0[8], qa1[8], qb0[8], qb1[8];
          auto rd = [&](int ks) {
            qa0[ks] = lds_tr4(ka0 + 16 * ks * D);
            qa1[ks] = lds_tr4(ka1 + 16 * ks * D);
            qb0[ks] = lds_tr4(db0 + 16 * ks * TR);
            qb1[ks] = lds_tr4(db1 + 16 * ks * TR);
          };
          rd(0);
          rd(1);
          f32x16 dq = zero16();
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) {
            if (ks + 2 < 8) rd(ks + 2);
            dq = mfma32(as_bf8(make_uint4(qa0[ks].x, qa0[ks].y, qa1[ks].x, qa1[ks].y)),
                        as_bf8(make_uint4(qb0[ks].x, qb0[ks].y, qb1[ks].x, qb1[ks].y)), dq);
          }
          // lane holds row l32, head-dim columns 32kq + 8j + 4h + (0..3); one lane
          // swap per dword gives lane half h whole 16-byte runs (columns 16pp + 8h .. +7)
          uint4 run[2];
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            const int e0 = 8 * pp, e1 = 8 * pp + 4;
            const auto s0 = __builtin_amdgcn_permlane32_swap(pack2(dq[e0], dq[e0 + 1]), pack2(dq[e1], dq[e1 + 1]),
                                                             false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(pack2(dq[e0 + 2], dq[e0 + 3]),
                                                             pack2(dq[e1 + 2], dq[e1 + 3]), false, false);
            run[pp] = make_uint4(s0[0], s1[0], s0[1], s1[1]);
          }
          const int p = rpair[qb][l32];  // the same for both lane halves of a row
          if (p >= 0) {  // runs 2k + h of head l32 % R, k = 2kq + pp, in the slot's run-interleaved layout
            bf16raw* dst = dq_part + (pair0 + (size_t)p) * R * D + 16 * (l32 % R) + 8 * h;
            st16nt(dst + 16 * R * (2 * kq), run[0]);
            st16nt(dst + 16 * R * (2 * kq + 1), run[1]);
          }
        }
      }
      __syncthreads();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    for (int i0 = -1; i0 < ntiles; i0 += 6) {  // i0 = -1 (mod 6): i0 + u has i mod 3 = (u+2)%3, i mod 2 = (u+1)%2
      consume(I2{}, I1{}, i0);
      consume(I0{}, I0{}, i0 + 1);
      consume(I1{}, I1{}, i0 + 2);
      consume(I2{}, I0{}, i0 + 3);
      consume(I0{}, I1{}, i0 + 4);
      consume(I1{}, I0{}, i0 + 5);
    }

    // ---- dK, dV of the owned keys and dims: lane holds head-dim column
    // 32(NCC dh + cc) + l32 of keys 64kh + 32kt + 8j + 4h + i.
    float* const dkb = dk_acc + kv0 * D;
    float* const dvb = dv_acc + kv0 * D;
    if (it.w & ITEM_SPLIT) {  // one of several items of this block: they run concurrently, so add atomically
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int kk = 64 * kh + 32 * kt + 8 * (e >> 2) + 4 * h + (e & 3);
            const int off = kk * G * D + 32 * (NCC * dh + cc) + l32;
            unsafeAtomicAdd(&dkb[off], dka[kt][cc][e]);
            unsafeAtomicAdd(&dvb[off], dva[kt][cc][e]);
          }
      return;
    }
    // The block's only item: per (key tile, dim tile), all 32 accumulator reads are issued before the stores.
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int cc = 0; cc < NCC; ++cc) {
        float ok[16], ov[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kk = 64 * kh + 32 * kt + 8 * (e >> 2) + 4 * h + (e & 3);
          const int off = kk * G * D + 32 * (NCC * dh + cc) + l32;
          ok[e] = dkb[off];
          ov[e] = dvb[off];
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kk = 64 * kh + 32 * kt + 8 * (e >> 2) + 4 * h + (e & 3);
          const int off = kk * G * D + 32 * (NCC * dh + cc) + l32;
          dkb[off] = ok[e] + dka[kt][cc][e];
          dvb[off] = ov[e] + dva[kt][cc][e];
        }
      }
  }
}

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

// dq[b,t,g*R+hh,:] = sum of the token's valid per-slot partials; one (batch,
// group, token) row per R*D/8 threads, 16 bytes per thread per slot.
template <int D, int R>
__global__ __launch_bounds__(256) void k_dq_combine(const int32_t* __restrict__ idx, const bf16raw* __restrict__ part,
                                                    bf16raw* __restrict__ dq, int T, int H, int G, int K, int t0,
                                                    int W, int rows) {
  constexpr int TPR = R * D / 8;
  constexpr int RPB = 256 / TPR;
  const int sub = threadIdx.x % TPR;
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= rows) return;
  const int bg = row / W, tl = row % W, t = t0 + tl, b = bg / G, g = bg % G;
  const int hh = sub / (D / 8), run = sub % (D / 8), c8 = run * 8;
  const int32_t* ir = idx + ((size_t)bg * T + t) * K;
  const size_t p0 = (size_t)bg * W * K + (size_t)tl * K;
  const unsigned last = (unsigned)(t / BLK);
  const bf16raw* pp = part + p0 * R * D + partial_run_offset<R>(hh, run);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  // slots per batch: independent loads in flight per thread.  32 covers a whole
  // row of topk 32 in one batch: two waves per SIMD issuing 32 loads each keep
  // more bytes in flight than seven waves issuing 8.
  constexpr int SB = 32;
  for (int s0 = 0; s0 < K; s0 += SB) {
    // entries and partial rows of the batch are loaded together; slots past K
    // re-read the last one and slots without a partial are masked after the load
    int ent[SB];
    uint4 raw[SB];
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int s = min(s0 + u, K - 1);
      ent[u] = ir[s];
      raw[u] = ld16nt(pp + (size_t)s * R * D);
    }
    // keep every load above the masking (the compiler would otherwise sink one
    // into a branch and issue it after the rest, costing a second round trip)
#pragma unroll
    for (int u = 0; u < SB; ++u) asm volatile("" : "+v"(raw[u].x), "+v"(raw[u].y), "+v"(raw[u].z), "+v"(raw[u].w));
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const bool ok = s0 + u < K && (unsigned)ent[u] <= last;
      raw[u] = ok ? raw[u] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const uint32_t wd[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        acc[2 * m] += __uint_as_float(wd[m] << 16);
        acc[2 * m + 1] += __uint_as_float(wd[m] & 0xffff0000u);
      }
    }
  }
  st16u(dq + ((size_t)(b * T + t) * H + g * R + hh) * D + c8,
        make_uint4(pack2(acc[0], acc[1]), pack2(acc[2], acc[3]), pack2(acc[4], acc[5]), pack2(acc[6], acc[7])));
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
  if ((long long)ib.max_items * g.B * g.G > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (const hipError_t e = launch_item_order(g, w, ib, st); e != hipSuccess) return e;
  dim3 grid(ib.max_items * g.B * g.G), block(BWD_THREADS);
  k_bwd_kv<D, R><<<grid, block, 0, st>>>(q, k, v, dout, lse, Dd, ib.items, ib.item_count, ib.list, ib.order, dq_part,
                                         dk_acc, dv_acc, g.T, g.H, g.G, g.K, w.t0, w.W, ib.max_items, g.scale,
                                         g.scale * LOG2E);
  return hipGetLastError();
}

template <int D, int R>
static hipError_t dq_combine_t(const Geo& g, const Win& w, const int32_t* idx, const uint16_t* dq_part, uint16_t* dq,
                               hipStream_t st) {
  const int rows = g.B * g.G * w.W;
  constexpr int RPB = 256 / (R * D / 8);
  k_dq_combine<D, R><<<(rows + RPB - 1) / RPB, 256, 0, st>>>(idx, dq_part, dq, g.T, g.H, g.G, g.K, w.t0, w.W,
                                                              rows);
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
