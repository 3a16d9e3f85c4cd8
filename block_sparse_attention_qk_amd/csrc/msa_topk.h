// Per-row top-k of pooled block scores, one row per wavefront, shared by the
// training-shape and decode-shape Index Branch kernels.
#pragma once
#include <climits>

#include "msa_common.h"

namespace msa {

// Top-k of one pooled row per wavefront.  Scores become order-preserving u32
// keys held in registers (VPL per lane).  The k-th largest key is found by a
// three-digit radix select (11, 11 and 10 bits): each digit is histogrammed in
// LDS over the keys that match the digits found so far, and a wave scan from
// the top bin finds the bin where the count of larger keys reaches k.  Blocks
// above the k-th key are taken, then blocks equal to it lowest index first;
// a ballot pass writes the chosen block ids in ascending order, and the row
// tail is -1.
constexpr int TOPK_BINS = 2048;

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
// in ascending block order and -1 to out[nsel..K).  `hist` is TOPK_BINS words
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

  uint32_t prefix = 0;
  int need = nsel;      // rank of the wanted key among keys matching prefix
  bool all_eq = false;  // every key equal to the final prefix is taken
  if constexpr (VPL <= 16) {
    // Short rows: build the k-th largest key bit by bit from the top; each
    // step is one ballot count per register of keys.  The bits that the row's
    // smallest and largest keys share are taken as they are (every key has
    // them), and the search stops once exactly nsel keys lie at or above the
    // prefix: the lower bits could then no longer change which keys are
    // chosen, and no unchosen key equals a chosen one.
    uint32_t kmin = 0xffffffffu, kmax = 0u;
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
    const uint32_t diff = kmin ^ kmax;
    int bit = diff == 0u ? -1 : 31 - __builtin_clz(diff);  // highest bit not shared by all keys
    prefix = bit < 0 ? kmax : (bit == 31 ? 0u : kmax & ~((2u << bit) - 1u));
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
  } else {
  // Radix select of the nsel-th largest key.  Pooled scores of a row share
  // their sign and exponent bits, so the digits start below the common prefix
  // of the row's smallest and largest key (otherwise every key would fall into
  // one histogram bin).
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    if (i * 64 >= nc) break;
    if (i * 64 + lane < nc) {
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
  }
  const uint32_t diff = kmin ^ kmax;
  int bits = diff == 0u ? 0 : 32 - __builtin_clz(diff);  // low bits still undecided
  prefix = bits == 32 ? 0u : (kmax & ~((1u << bits) - 1u));
  while (bits > 0) {
    const int width = bits < 11 ? bits : 11;
    const int sh = bits - width, nbins = 1 << width;
    const uint32_t hi_mask = bits == 32 ? 0u : ~((1u << bits) - 1u);
    for (int j = lane; j < nbins; j += 64) hist[j] = 0;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      if (i * 64 >= nc) break;
      if (i * 64 + lane < nc && (key[i] & hi_mask) == prefix)
        atomicAdd(&hist[(key[i] >> sh) & (nbins - 1)], 1u);
    }
    __builtin_amdgcn_wave_barrier();
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
    uint32_t cbin = 0;  // keys in the chosen bin
    for (int j = 0; j < per; ++j) {  // every lane walks the owner's bins (LDS broadcast)
      const uint32_t c = hist[otop - 1 - j];
      if (run + c >= (uint32_t)need) {
        bin = otop - 1 - j;
        cbin = c;
        break;
      }
      run += c;
    }
    need -= (int)run;
    prefix |= (uint32_t)bin << sh;
    bits = sh;
    // The chosen bin holds exactly the keys still needed: all of them are taken,
    // the lower digits cannot change that, and no other key ties with them.
    if (cbin == (uint32_t)need) {
      all_eq = true;
      break;
    }
    __builtin_amdgcn_wave_barrier();
  }
  }
  const uint32_t kth = prefix;
  const int need_eq = all_eq ? INT_MAX : need;  // equal keys to take, lowest block index first

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
