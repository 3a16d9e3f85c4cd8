// Decode step for gfx950: one new query per sequence against its caches.
//
// ai-beat "flash-msa-sparse-attention-training", paragraph 1: MSA is served
// for inference as well (prefill and decode).  A decode step computes, for the
// new token at position t = len - 1 of each sequence, exactly what the
// training path computes for row t: the proxy query is scored against every
// cached causal proxy key, the scores are max-pooled per 128-key block, the
// top-k blocks are kept (xcelit "Flash-MSA: Open-Source Sparse Attention
// Kernels Debut", section "How MSA works"), and exact softmax attention runs
// over the keys of those blocks only.
//
// Both halves are bound by HBM reads (the proxy-key cache, then the selected
// K/V blocks), so the kernels are laid out for streaming: 16-byte coalesced
// loads with many in flight per lane, and enough workgroups to cover the chip
// even for a single sequence.  QK^T runs on v_mfma_f32_32x32x16_bf16 because
// cached K rows are contiguous along the contraction; P V is a plain FMA loop
// in which each lane owns two value columns for all heads of its group.
#include "msa_common.h"
#include "msa_internal.h"
#include "msa_topk.h"

namespace msa {

constexpr int DEC_WAVES = 4;  // waves per workgroup in the decode kernels

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// sum_i q[i] * x[i] over the eight bf16 values packed in r (fp32 products and sums)
__device__ __forceinline__ float dot8(const float* q, const uint4& r) {
  float s = q[0] * bf_lo(r.x);
  s = fmaf(q[1], bf_hi(r.x), s);
  s = fmaf(q[2], bf_lo(r.y), s);
  s = fmaf(q[3], bf_hi(r.y), s);
  s = fmaf(q[4], bf_lo(r.z), s);
  s = fmaf(q[5], bf_hi(r.z), s);
  s = fmaf(q[6], bf_lo(r.w), s);
  s = fmaf(q[7], bf_hi(r.w), s);
  return s;
}

// Proxy scores of the new query against the cached proxy keys of one block,
// max-pooled.  One wave streams one 128-token block for GS consecutive groups:
// a token's GS groups are CPT = GS*DP/8 16-byte chunks, a wave load covers
// 64/CPT tokens, and the DP/8 lanes of one (token, group) add their partial
// dot products with xor shuffles before the running max.  Tokens past the new
// one are never read (their loads are clamped to the last cached row and their
// scores dropped).
template <int DP, int GS>
__global__ __launch_bounds__(64 * DEC_WAVES) void k_dec_pool(const bf16raw* __restrict__ qp,
                                                             const bf16raw* __restrict__ kp,
                                                             const int32_t* __restrict__ len,
                                                             float* __restrict__ pooled, int T, int G, int N) {
  constexpr int CPG = DP / 8;
  constexpr int CPT = GS * CPG;
  static_assert(CPT <= 64 && 64 % CPT == 0, "a token's chunks must tile a wave");
  constexpr int TPL = 64 / CPT;
  constexpr int LOADS = BLK / TPL;
  constexpr int U = LOADS < 16 ? LOADS : 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ngs = G / GS;
  const int b = blockIdx.y / ngs, g0 = (blockIdx.y % ngs) * GS;
  const int blk = blockIdx.x * DEC_WAVES + wave;
  const int L = len[b];
  if (L < 1 || L > T) return;  // whole wave
  const int t = L - 1;
  if (blk > t / BLK) return;  // whole wave
  const int tok = lane / CPT, c = lane % CPT, gg = c / CPG;
  float q[8];
  {
    const uint4 r = ld16u(qp + ((size_t)b * G + g0) * DP + c * 8);
    q[0] = bf_lo(r.x); q[1] = bf_hi(r.x); q[2] = bf_lo(r.y); q[3] = bf_hi(r.y);
    q[4] = bf_lo(r.z); q[5] = bf_hi(r.z); q[6] = bf_lo(r.w); q[7] = bf_hi(r.w);
  }
  const int jmax = t - blk * BLK;  // in-block offsets 0..jmax are causal
  const size_t rs = (size_t)G * DP;  // elements per cached token
  const bf16raw* src = kp + ((size_t)b * T + (size_t)blk * BLK) * rs + (size_t)g0 * DP + c * 8;
  float m = -INFINITY;
  for (int i0 = 0; i0 < LOADS; i0 += U) {
    uint4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = ld16nt(src + (size_t)min((i0 + u) * TPL + tok, jmax) * rs);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float s = dot8(q, r[u]);
#pragma unroll
      for (int off = 1; off < CPG; off <<= 1) s += __shfl_xor(s, off);
      if ((i0 + u) * TPL + tok <= jmax) m = fmaxf(m, s);
    }
  }
#pragma unroll
  for (int off = CPT; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (tok == 0 && c % CPG == 0) pooled[((size_t)b * G + g0 + gg) * N + blk] = m;
}

// Top-k of each (sequence, group) pooled row with the rule of the training
// rows (min(K, t/128 + 1) blocks, ties to the lower index, ascending, -1 tail),
// one 1024-thread workgroup per row: decode has few rows, so the whole
// workgroup shares one row.  Thread i holds the order-preserving keys of
// blocks i, i + 1024, ...; the k-th largest key comes from a radix select over
// digits of the bits below the row's common prefix (histograms in LDS, the bin
// found by one wave's scan); the chosen blocks are then written in ascending
// order by a workgroup prefix count.  Sequences whose length is outside 1..T
// get an all -1 row.
constexpr int DTK_THREADS = 1024;
constexpr int DTK_WAVES = DTK_THREADS / 64;

template <int VPT>
__global__ __launch_bounds__(DTK_THREADS) void k_dec_topk(const float* __restrict__ pooled,
                                                          const int32_t* __restrict__ len, int32_t* __restrict__ idx,
                                                          int T, int G, int N, int K) {
  __shared__ uint32_t hist[TOPK_BINS];
  __shared__ uint32_t red[2][DTK_WAVES];
  __shared__ int bc[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;
  const int L = len[row / G];
  int32_t* out = idx + (size_t)row * K;
  if (L < 1 || L > T) {
    for (int p = tid; p < K; p += DTK_THREADS) out[p] = -1;
    return;  // whole workgroup
  }
  const int nc = (L - 1) / BLK + 1, nsel = min(K, nc);
  const float* pr = pooled + (size_t)row * N;
  // All loads in flight together: columns past the causal blocks read the
  // last causal score (nc >= 1) and are masked after.
  float sc[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) sc[i] = pr[min(i * DTK_THREADS + tid, nc - 1)];
  uint32_t key[VPT];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const bool valid = i * DTK_THREADS + tid < nc;
    const uint32_t kk = valid ? score_key(sc[i]) : 0u;
    kmin = valid ? min(kmin, kk) : kmin;
    kmax = valid ? max(kmax, kk) : kmax;
    key[i] = kk;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
  }
  if (lane == 0) {
    red[0][wave] = kmin;
    red[1][wave] = kmax;
  }
  __syncthreads();
  kmin = 0xffffffffu;
  kmax = 0u;
#pragma unroll
  for (int w = 0; w < DTK_WAVES; ++w) {
    kmin = min(kmin, red[0][w]);
    kmax = max(kmax, red[1][w]);
  }
  // Radix select of the nsel-th largest key below the common prefix of kmin and kmax.
  const uint32_t diff = kmin ^ kmax;
  int bits = diff == 0u ? 0 : 32 - __builtin_clz(diff);
  uint32_t prefix = bits == 32 ? 0u : (kmax & ~((1u << bits) - 1u));
  int need = nsel;  // rank of the wanted key among the keys matching prefix
  while (bits > 0) {
    const int width = bits < 11 ? bits : 11;
    const int sh = bits - width, nbins = 1 << width;
    const uint32_t hi_mask = bits == 32 ? 0u : ~((1u << bits) - 1u);
    for (int j = tid; j < nbins; j += DTK_THREADS) hist[j] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < VPT; ++i)
      if (i * DTK_THREADS + tid < nc && (key[i] & hi_mask) == prefix) atomicAdd(&hist[(key[i] >> sh) & (nbins - 1)], 1u);
    __syncthreads();
    if (wave == 0) {
      // lanes own `per` consecutive bins each, scanned from the top bin down
      const int per = nbins >= 64 ? nbins / 64 : 1;
      const int top = nbins - per * lane;
      uint32_t lsum = 0;
      if (top > 0)
        for (int j = 0; j < per; ++j) lsum += hist[top - 1 - j];
      uint32_t incl = lsum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      const uint32_t excl = incl - lsum;
      const unsigned long long hit = __ballot(top > 0 && excl < (uint32_t)need && (uint32_t)need <= incl);
      const int owner = __builtin_ctzll(hit);
      uint32_t run = __shfl(excl, owner);
      const int otop = nbins - per * owner;
      int bin = otop - 1;
      for (int j = 0; j < per; ++j) {
        const uint32_t c = hist[otop - 1 - j];
        if (run + c >= (uint32_t)need) {
          bin = otop - 1 - j;
          break;
        }
        run += c;
      }
      if (lane == 0) {
        bc[0] = bin;
        bc[1] = need - (int)run;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)bc[0] << sh;
    need = bc[1];
    bits = sh;
    __syncthreads();  // bc and hist are rewritten by the next digit
  }
  const uint32_t kth = prefix;
  const int need_eq = need;  // keys equal to kth to take, lowest block index first
  // Ascending write-out: blocks in column order i * 1024 + tid, ranks from
  // per-wave ballots and a prefix over the waves.
  const unsigned long long lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int base_eq = 0, base_sel = 0;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int col = i * DTK_THREADS + tid;
    const bool valid = col < nc;
    const bool eq = valid && key[i] == kth, gt = valid && key[i] > kth;
    const unsigned long long meq = __ballot(eq);
    if (lane == 0) red[0][wave] = (uint32_t)__popcll(meq);
    __syncthreads();
    int eq_before = base_eq, eq_total = 0;
#pragma unroll
    for (int w = 0; w < DTK_WAVES; ++w) {
      const int c = (int)red[0][w];
      if (w < wave) eq_before += c;
      eq_total += c;
    }
    const bool sel = gt || (eq && eq_before + (int)__popcll(meq & lt) < need_eq);
    const unsigned long long msel = __ballot(sel);
    if (lane == 0) red[1][wave] = (uint32_t)__popcll(msel);
    __syncthreads();
    int sel_before = base_sel, sel_total = 0;
#pragma unroll
    for (int w = 0; w < DTK_WAVES; ++w) {
      const int c = (int)red[1][w];
      if (w < wave) sel_before += c;
      sel_total += c;
    }
    if (sel) out[sel_before + __popcll(msel & lt)] = col;
    base_eq += eq_total;
    base_sel += sel_total;
    __syncthreads();  // red is rewritten by the next column group
  }
  for (int p = nsel + tid; p < K; p += DTK_THREADS) out[p] = -1;
}

// Attention of the new query's R heads over one selected block (one workgroup
// per (sequence, group, slot)); the four waves take 32 keys each.
//   S^T (32 keys x 32 columns, R used) = K_rows . Q^T on 32x32x16 MFMA;
//   per wave: max, exp2, row sums; P goes to LDS as [key][head];
//   P V: lane owns two value columns for all R heads (for d = 64 the two
//   halves of the wave take alternate keys and are summed at the end);
//   the four waves' (max, sum, PV) merge in LDS into one normalised partial
//   o (fp32, [R][d]) and its natural-log lse per head.
// Slots that are empty (-1) or not causal for this length are skipped; the
// combine skips them too.  Key rows past the new token are never read: the
// loads are clamped to the last cached row and their probabilities are zero.
template <int D, int R>
__global__ __launch_bounds__(64 * DEC_WAVES) void k_dec_attn(const bf16raw* __restrict__ q,
                                                             const bf16raw* __restrict__ k,
                                                             const bf16raw* __restrict__ v,
                                                             const int32_t* __restrict__ len,
                                                             const int32_t* __restrict__ idx,
                                                             float* __restrict__ part_o, float* __restrict__ part_lse,
                                                             int T, int G, int K, float scale_log2) {
  static_assert(R <= 32, "heads per group must fit the 32 MFMA columns");
  constexpr int KH = 128 / D;  // wave halves splitting the keys in P V (2 for d = 64)
  __shared__ float Ps[DEC_WAVES][32][R];
  __shared__ float Ms[DEC_WAVES][R], Ls[DEC_WAVES][R];
  __shared__ float Os[DEC_WAVES][R][D];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = blockIdx.x, bg = blockIdx.y, b = bg / G, g = bg % G;
  const int L = len[b];
  if (L < 1 || L > T) return;  // whole workgroup
  const int t = L - 1;
  const int blk = idx[(size_t)bg * K + slot];
  if (blk < 0 || blk > t / BLK) return;  // whole workgroup
  const int H = G * R;
  const int kbase = blk * BLK + 32 * wave;

  // ---- S^T = K Q^T: A = K rows (lane: key lane%32, 8 dims at 8*(lane/32) of each 16-dim step),
  // B = Q^T (lane: head lane%32, same dims; zero for heads >= R)
  const int h = lane & 31, half = lane >> 5;
  const bool hv = h < R;
  const bf16raw* krow = k + (((size_t)b * T + min(kbase + h, t)) * G + g) * D + 8 * half;
  const bf16raw* qrow = q + ((size_t)b * H + g * R + (hv ? h : 0)) * D + 8 * half;
  bf16x8 ka[D / 16], qb[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    ka[st] = ld8(krow + 16 * st);
    qb[st] = ld8(qrow + 16 * st);
  }
  // Value rows for P V (lane: two columns c0, c0 + 1 of keys kbase + i*KH + kh), issued
  // together with the K rows so that both HBM round trips overlap.
  const int c0 = 2 * (lane % (D / 2));
  const int kh = lane / (D / 2);  // 0 for d = 128
  uint32_t vv[32 / KH];
#pragma unroll
  for (int i = 0; i < 32 / KH; ++i) {
    const int key = min(kbase + i * KH + kh, t);
    vv[i] = *reinterpret_cast<const uint32_t*>(v + (((size_t)b * T + key) * G + g) * D + c0);
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x16 acc = zero16();
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    bf16x8 bq = qb[st];
    if (!hv) bq = as_bf8(make_uint4(0u, 0u, 0u, 0u));
    acc = mfma32(ka[st], bq, acc);
  }
  // lane holds head h, keys kbase + 8*(e/4) + 4*half + e%4
  float s[16];
  float mw = -INFINITY;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int key = kbase + 8 * (e >> 2) + 4 * half + (e & 3);
    s[e] = key <= t ? acc[e] * scale_log2 : -INFINITY;
    mw = fmaxf(mw, s[e]);
  }
  mw = fmaxf(mw, __shfl_xor(mw, 32));
  float lw = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float p = mw == -INFINITY ? 0.f : fast_exp2(s[e] - mw);
    lw += p;
    if (hv) Ps[wave][8 * (e >> 2) + 4 * half + (e & 3)][h] = p;
  }
  lw += __shfl_xor(lw, 32);
  if (hv && half == 0) {
    Ms[wave][h] = mw;
    Ls[wave][h] = lw;
  }
  // The P V loop below reads only this wave's rows of Ps: a wave's LDS accesses complete in
  // order, so the wave barrier (which keeps the compiler from moving accesses across it) suffices.
  __builtin_amdgcn_wave_barrier();

  // ---- P V over the wave's 32 keys
  float o0[R], o1[R];
#pragma unroll
  for (int r = 0; r < R; ++r) o0[r] = o1[r] = 0.f;
#pragma unroll
  for (int i = 0; i < 32 / KH; ++i) {
    const float v0 = bf_lo(vv[i]), v1 = bf_hi(vv[i]);
    const float* pr = Ps[wave][i * KH + kh];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      o0[r] = fmaf(pr[r], v0, o0[r]);
      o1[r] = fmaf(pr[r], v1, o1[r]);
    }
  }
  if (KH == 2) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      o0[r] += __shfl_xor(o0[r], 32);
      o1[r] += __shfl_xor(o1[r], 32);
    }
  }
  if (kh == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) *reinterpret_cast<float2*>(&Os[wave][r][c0]) = make_float2(o0[r], o1[r]);
  }
  __syncthreads();

  // ---- merge the four waves into the slot's partial
  float* po = part_o + ((size_t)bg * K + slot) * R * D;
  float* pl = part_lse + ((size_t)bg * K + slot) * R;
  for (int x = threadIdx.x; x < R * D; x += 64 * DEC_WAVES) {
    const int hh = x / D, cc = x % D;
    float M = Ms[0][hh];
#pragma unroll
    for (int w = 1; w < DEC_WAVES; ++w) M = fmaxf(M, Ms[w][hh]);
    float sl = 0.f, so = 0.f;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) {
      const float f = Ms[w][hh] == -INFINITY ? 0.f : fast_exp2(Ms[w][hh] - M);
      sl = fmaf(f, Ls[w][hh], sl);
      so = fmaf(f, Os[w][hh][cc], so);
    }
    po[x] = so / sl;
    if (cc == 0) pl[hh] = (M + fast_log2(sl)) * 0.6931471805599453f;
  }
}

// Log-sum-exp merge of the slot partials of one (sequence, head): NW waves
// per head (4, or 16 for long rows), wave w taking slots w, w + NW, ...  The
// workgroup first finds the
// max of the valid slots' lse, then every lane adds the weighted partials of
// its D/64 value columns over its wave's slots (the loads do not depend on each
// other), and the NW sums meet in LDS.  Rows with no valid slot (length
// outside 1..T) get o = 0 and lse = -inf; rows with a NaN slot lse get NaN.
template <int D, int R, int DCB_WAVES>
__global__ __launch_bounds__(64 * DCB_WAVES) void k_dec_combine(const float* __restrict__ part_o,
                                                                const float* __restrict__ part_lse,
                                                                const int32_t* __restrict__ idx,
                                                                const int32_t* __restrict__ len,
                                                                bf16raw* __restrict__ o, float* __restrict__ lse,
                                                                int T, int G, int K) {
  constexpr int CL = D / 64;  // value columns per lane
  __shared__ float red[DCB_WAVES];
  __shared__ int red_nan[DCB_WAVES];
  __shared__ float acc[DCB_WAVES][D + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bh = blockIdx.x, H = G * R, b = bh / H, h = bh % H, g = h / R, hh = h % R;
  const int bg = b * G + g;
  const int L = len[b];
  const int nb = (L >= 1 && L <= T) ? (L - 1) / BLK + 1 : 0;  // causal blocks; 0 = no valid slot
  const int32_t* row = idx + (size_t)bg * K;
  const float* pl = part_lse + (size_t)bg * K * R + hh;
  const float* po = part_o + ((size_t)bg * K * R + hh) * D + CL * lane;
  float M = -INFINITY;
  bool nan_seen = false;  // a NaN slot lse (skipped by the max) makes the row NaN
  for (int sl = threadIdx.x; sl < K; sl += 64 * DCB_WAVES) {
    const int blk = row[sl];
    if (blk >= 0 && blk < nb) {
      const float x = pl[(size_t)sl * R];
      M = fmaxf(M, x);
      nan_seen |= x != x;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  nan_seen = __any(nan_seen);
  if (lane == 0) {
    red[wave] = M;
    red_nan[wave] = nan_seen;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < DCB_WAVES; ++w) {
    M = fmaxf(M, red[w]);
    nan_seen |= red_nan[w] != 0;
  }
  float sw = 0.f, so[CL];
#pragma unroll
  for (int c = 0; c < CL; ++c) so[c] = 0.f;
  if (M != -INFINITY) {
#pragma unroll 4
    for (int sl = wave; sl < K; sl += DCB_WAVES) {
      const int blk = row[sl];
      const bool ok = blk >= 0 && blk < nb;
      const float w = ok ? __expf(pl[(size_t)sl * R] - M) : 0.f;
      sw += w;
      const float* src = po + (size_t)sl * R * D;
#pragma unroll
      for (int c = 0; c < CL; ++c) so[c] = fmaf(w, ok ? src[c] : 0.f, so[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < CL; ++c) acc[wave][CL * lane + c] = so[c];
  if (lane == 0) acc[wave][D] = sw;
  __syncthreads();
  if (wave != 0) return;
  float tw = 0.f;
#pragma unroll
  for (int w = 0; w < DCB_WAVES; ++w) tw += acc[w][D];
  const size_t oh = (size_t)b * H + h;
#pragma unroll
  for (int c = 0; c < CL; ++c) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < DCB_WAVES; ++w) v += acc[w][CL * lane + c];
    o[oh * D + CL * lane + c] = f2bf(nan_seen ? __builtin_nanf("") : M == -INFINITY ? 0.f : v / tw);
  }
  if (lane == 0) lse[oh] = nan_seen ? __builtin_nanf("") : M == -INFINITY ? -INFINITY : M + __logf(tw);
}

// ---- host launchers

static int pool_gs(int G, int DP) {
  int gs = 1;
  while (G % (2 * gs) == 0 && 2 * gs * DP <= 512) gs *= 2;
  return gs;
}

hipError_t launch_dec_pool(const Geo& g, const uint16_t* qp, const uint16_t* kp, const int32_t* len, float* pooled,
                           hipStream_t st) {
  const int gs = pool_gs(g.G, g.DP);
  dim3 grid((g.N + DEC_WAVES - 1) / DEC_WAVES, g.B * (g.G / gs)), block(64 * DEC_WAVES);
#define MSA_DEC_POOL(DPV, GSV)                                                         \
  if (g.DP == DPV && gs == GSV) {                                                      \
    k_dec_pool<DPV, GSV><<<grid, block, 0, st>>>(qp, kp, len, pooled, g.T, g.G, g.N);  \
    return hipGetLastError();                                                          \
  }
  MSA_DEC_POOL(32, 1) MSA_DEC_POOL(32, 2) MSA_DEC_POOL(32, 4) MSA_DEC_POOL(32, 8) MSA_DEC_POOL(32, 16)
  MSA_DEC_POOL(64, 1) MSA_DEC_POOL(64, 2) MSA_DEC_POOL(64, 4) MSA_DEC_POOL(64, 8)
  MSA_DEC_POOL(128, 1) MSA_DEC_POOL(128, 2) MSA_DEC_POOL(128, 4)
#undef MSA_DEC_POOL
  return hipErrorInvalidValue;
}

hipError_t launch_dec_topk(const Geo& g, const float* pooled, const int32_t* len, int32_t* idx, hipStream_t st) {
  const int rows = g.B * g.G;
  const int need = (g.N + DTK_THREADS - 1) / DTK_THREADS;
#define MSA_DEC_TOPK(V)                                                                       \
  if (need <= V) {                                                                            \
    k_dec_topk<V><<<dim3(rows), dim3(DTK_THREADS), 0, st>>>(pooled, len, idx, g.T, g.G, g.N, g.K); \
    return hipGetLastError();                                                                 \
  }
  MSA_DEC_TOPK(1)
  MSA_DEC_TOPK(2)
  MSA_DEC_TOPK(4)
  MSA_DEC_TOPK(8)
#undef MSA_DEC_TOPK
  return hipErrorInvalidValue;
}

hipError_t launch_dec_attn(const Geo& g, const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* len,
                           const int32_t* idx, float* part_o, float* part_lse, hipStream_t st) {
  dim3 grid(g.K, g.B * g.G), block(64 * DEC_WAVES);
  const float sl2 = g.scale * 1.4426950408889634f;
#define MSA_DEC_ATTN(DV, RV)                                                                                     \
  if (g.D == DV && g.R == RV) {                                                                                  \
    k_dec_attn<DV, RV><<<grid, block, 0, st>>>(q, k, v, len, idx, part_o, part_lse, g.T, g.G, g.K, sl2);       \
    return hipGetLastError();                                                                                    \
  }
  MSA_DEC_ATTN(64, 1) MSA_DEC_ATTN(64, 2) MSA_DEC_ATTN(64, 4) MSA_DEC_ATTN(64, 8) MSA_DEC_ATTN(64, 16)
  MSA_DEC_ATTN(128, 1) MSA_DEC_ATTN(128, 2) MSA_DEC_ATTN(128, 4) MSA_DEC_ATTN(128, 8) MSA_DEC_ATTN(128, 16)
#undef MSA_DEC_ATTN
  return hipErrorInvalidValue;
}

hipError_t launch_dec_combine(const Geo& g, const float* part_o, const float* part_lse, const int32_t* idx,
                              const int32_t* len, uint16_t* o, float* lse, hipStream_t st) {
  const bool wide = g.K >= 128;  // long rows: 16 waves share a head's slots
  dim3 grid(g.B * g.H), block(wide ? 1024 : 256);
#define MSA_DEC_COMB(DV, RV)                                                                                     \
  if (g.D == DV && g.R == RV) {                                                                                  \
    if (wide)                                                                                                    \
      k_dec_combine<DV, RV, 16><<<grid, block, 0, st>>>(part_o, part_lse, idx, len, o, lse, g.T, g.G, g.K);     \
    else                                                                                                         \
      k_dec_combine<DV, RV, 4><<<grid, block, 0, st>>>(part_o, part_lse, idx, len, o, lse, g.T, g.G, g.K);      \
    return hipGetLastError();                                                                                    \
  }
  MSA_DEC_COMB(64, 1) MSA_DEC_COMB(64, 2) MSA_DEC_COMB(64, 4) MSA_DEC_COMB(64, 8) MSA_DEC_COMB(64, 16)
  MSA_DEC_COMB(128, 1) MSA_DEC_COMB(128, 2) MSA_DEC_COMB(128, 4) MSA_DEC_COMB(128, 8) MSA_DEC_COMB(128, 16)
#undef MSA_DEC_COMB
  return hipErrorInvalidValue;
}

}  // namespace msa
