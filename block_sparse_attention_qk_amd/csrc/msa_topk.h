// Per-row top-k of pooled block scores: the order-preserving score keys and
// histogram sizes shared by the training and decode Index Branch kernels, and
// the one-wave-per-row routine of the training kernel for rows up to 1024 blocks.
#pragma once
#include <climits>

#include "msa_common.h"

namespace msa {

// Top-k of one pooled row per wavefront (rows of at most 1024 blocks).  Scores
// become order-preserving u32 keys held in registers (VPL per lane).  The k-th
// largest key is found from a histogram of 256 bins spread linearly between
// the row's smallest and largest score: the chosen bin's few keys are ranked
// directly.  Rows with non-finite or equal extreme scores, or a crowded bin,
// build the k-th key bit by bit instead.  Blocks above the k-th key are taken,
// then blocks equal to it lowest index first; a ballot pass writes the chosen
// block ids in ascending order, and the row tail is -1.
constexpr int TOPK_BINS = 2048;
constexpr int TOPK_LIN_BINS = 256;                     // linear first digit of rows up to 1024 blocks
constexpr int TOPK_ROW_LDS = TOPK_LIN_BINS + 64;        // LDS words per wave: bins, then the chosen bin's keys

// Order-preserving u32 key of a score; -0 ranks equal to +0.
__device__ __forceinline__ uint32_t score_key(float f) {
  if (f == 0.0f) f = 0.0f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The score of a key (the inverse of score_key; -0 comes back as +0).
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Writes the nsel = min(K, nc) best of the nc scores pr[0..nc) to out[0..nsel)
// in ascending block order and -1 to out[nsel..K).  `hist` is TOPK_ROW_LDS words
// of this wave's LDS.  All 64 lanes must call it together.
template <int VPL>
__device__ __forceinline__ void topk_row(const float* __restrict__ pr, int nc, int K, int32_t* __restrict__ out,
                                         uint32_t* hist, int lane) {
  const int nsel = min(K, nc);

  // Every load is issued before the first is used: columns past the row's
  // causal blocks read its last causal score (nc >= 1) and are masked after.
  float sc[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) sc[i] = pr[min(i * 64 + lane, nc - 1)];
  uint32_t key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) key[i] = i * 64 + lane < nc ? score_key(sc[i]) : 0u;

  static_assert(VPL <= 16, "rows of more than 1024 blocks take the workgroup kernel");
  uint32_t prefix = 0;
  int need = nsel;  // equal keys to take, lowest block index first
  uint32_t kmin = 0xffffffffu, kmax = 0u;  // over the row's causal blocks
#pragma unroll
  for (int i = 0; i < VPL; ++i)
    if (i * 64 + lane < nc) {
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
    }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
  }
  // First, when the row's scores are finite and not all equal: 256 bins
  // spread linearly between its smallest and largest score.  The bin is a
  // non-decreasing function of the score, so the k-th key lies in the chosen
  // bin and every key of a higher bin is larger; the chosen bin holds a few
  // keys, ranked directly.  A row that takes every causal block needs no
  // search (its k-th key is the smallest).
  bool found = nsel == nc;
  if (found) prefix = kmin;
  const float fmin = key_score(kmin), fmax = key_score(kmax);
  const float span = fmax - fmin, scl = (float)TOPK_LIN_BINS / span;
  if (!found && fmax > fmin && __builtin_isfinite(span) && __builtin_isfinite(scl) && scl > 0.f) {
    constexpr int PERL = TOPK_LIN_BINS / 64;  // bins per lane in the scan
    int lb[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      lb[i] = i * 64 + lane < nc ? min(TOPK_LIN_BINS - 1, (int)((sc[i] - fmin) * scl)) : -1;
#pragma unroll
    for (int j = 0; j < PERL; ++j) hist[lane + 64 * j] = 0;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lb[i] >= 0) atomicAdd(&hist[lb[i]], 1u);
    __builtin_amdgcn_wave_barrier();
    // lane owns bins [top - PERL, top) counted from the top bin down
    const int top = TOPK_LIN_BINS - PERL * lane;
    uint32_t c[PERL], lsum = 0;
#pragma unroll
    for (int j = 0; j < PERL; ++j) {
      c[j] = hist[top - 1 - j];
      lsum += c[j];
    }
    uint32_t incl = lsum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    const uint32_t excl = incl - lsum;
    int bin = -1, nb = 0, cb = 0;  // chosen bin, rank of the k-th key in it, its count (owner lane)
    if (excl < (uint32_t)nsel && (uint32_t)nsel <= incl) {
      uint32_t run = excl;
#pragma unroll
      for (int j = 0; j < PERL; ++j) {
        if (bin < 0 && run + c[j] >= (uint32_t)nsel) {
          bin = top - 1 - j;
          nb = nsel - (int)run;
          cb = (int)c[j];
        }
        run += c[j];
      }
    }
    const int owner = __builtin_ctzll(__ballot(bin >= 0));
    bin = __shfl(bin, owner);
    nb = __shfl(nb, owner);
    cb = __shfl(cb, owner);
    if (cb <= 64) {  // gather the bin's keys after the bins, then rank them
      uint32_t* cand = hist + TOPK_LIN_BINS;
      const unsigned long long lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
      int base = 0;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const unsigned long long m = __ballot(lb[i] == bin);
        if (lb[i] == bin) cand[base + __popcll(m & lt)] = key[i];
        base += __popcll(m);
      }
      __builtin_amdgcn_wave_barrier();
      bool hit = false;
      uint32_t mine = 0u;
      if (lane < cb) {  // the key with fewer than nb larger and at least nb at least as large
        mine = cand[lane];
        int gt = 0, ge = 0;
        for (int j = 0; j < cb; ++j) {
          const uint32_t o = cand[j];
          gt += o > mine;
          ge += o >= mine;
        }
        hit = gt < nb && nb <= ge;
      }
      const unsigned long long hm = __ballot(hit);
      if (hm != 0ull) {
        prefix = (uint32_t)__shfl((int)mine, __builtin_ctzll(hm));
        found = true;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  // Otherwise build the k-th largest key bit by bit from the top; each step
  // is one ballot count per register of keys.  The bits that the row's
  // smallest and largest keys share are taken as they are (every key has
  // them), and the search stops once exactly nsel keys lie at or above the
  // prefix: the lower bits could then no longer change which keys are
  // chosen, and no unchosen key equals a chosen one.
  const uint32_t diff = kmin ^ kmax;
  int bit = found ? -1 : (diff == 0u ? -1 : 31 - __builtin_clz(diff));  // highest bit not shared by all keys
  if (!found) prefix = bit < 0 ? kmax : (bit == 31 ? 0u : kmax & ~((2u << bit) - 1u));
  int cge = nc;  // keys at or above prefix
  for (; bit >= 0 && cge != nsel; --bit) {
    const uint32_t cand = prefix | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (i * 64 < nc) cnt += __popcll(__ballot((i * 64 + lane < nc) && key[i] >= cand));
    if (cnt >= nsel) {
      prefix = cand;
      cge = cnt;
    }
  }
  int cnt_gt = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i)
    if (i * 64 < nc) cnt_gt += __popcll(__ballot((i * 64 + lane < nc) && key[i] > prefix));
  need = nsel - cnt_gt;
  const uint32_t kth = prefix;
  const int need_eq = need;

  const unsigned long long lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int run_eq = 0, run_sel = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    if (i * 64 >= nc) break;
    const bool valid = i * 64 + lane < nc;
    const bool eq = valid && key[i] == kth, gt = valid && key[i] > kth;
    const unsigned long long meq = __ballot(eq);
    const int rank = run_eq + __popcll(meq & lt);
    const bool sel = gt || (eq && rank < need_eq);
    const unsigned long long msel = __ballot(sel);
    if (sel) out[run_sel + __popcll(msel & lt)] = i * 64 + lane;
    run_eq += __popcll(meq);
    run_sel += __popcll(msel);
  }
  for (int p = nsel + lane; p < K; p += 64) out[p] = -1;
}

}  // namespace msa
