// Index Branch kernels for gfx950: proxy score + 128-key block max-pool, and
// the per-row top-k that fills the block-index cache.
//
// Method (pages: xcelit "Flash-MSA: Open-Source Sparse Attention Kernels
// Debut", section "How MSA works"; ai-beat "flash-msa-sparse-attention-
// training", paragraphs 1, 3, 4): one proxy head per KV group scores every
// query against every causal key, scores are max-pooled over 128-key blocks,
// and the top-k blocks per query are cached.  This is the only quadratic step.
#include "msa_common.h"
#include "msa_internal.h"

namespace msa {

constexpr int POOL_QT = 256;   // queries per workgroup (4 waves x 64)
constexpr int POOL_CHB = 16;   // pooled blocks buffered in LDS between flushes

// Pooled scores for the queries [t0, t0+W) of one (batch, group):
//   pooled[(bg*W + t - t0)*N + i] = max_{128i <= j <= min(128i+127, t)} qp[t].kp[j]
// for i <= t/128 (other entries are not written).
//
// Each wave owns 64 queries (4 MFMA column tiles) whose proxy rows stay in
// registers as B operands.  Key blocks stream through a double-buffered LDS
// tile; the product is taken transposed (S^T = Kp Qp^T, keys along M) so that a
// lane holds 32 keys of one query column: the block max is 31 in-lane maxima
// and two cross-lane steps.  Pooled values collect in LDS and leave as 64-byte
// row segments.
template <int DP>
__global__ __launch_bounds__(256, 2) void k_proxy_pool(const bf16raw* __restrict__ qp,
                                                       const bf16raw* __restrict__ kp,
                                                       float* __restrict__ pooled, int T, int G, int N,
                                                       int t0, int W) {
  constexpr int KS = DP / 32;      // MFMA k-steps over the proxy dim
  constexpr int LDK = DP + 8;      // LDS row stride in bf16 (keeps 16 rows on distinct banks)
  constexpr int CPT = DP / 16;     // 16-byte chunks per thread per key block
  __shared__ __attribute__((aligned(16))) bf16raw kbuf[2][BLK * LDK];
  __shared__ float pbuf[POOL_QT * (POOL_CHB + 1)];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int bg = blockIdx.y, b = bg / G, g = bg % G;
  const int tile = gridDim.x - 1 - blockIdx.x;  // longest rows first
  const int qt0 = t0 + tile * POOL_QT;
  const int qlast = min(qt0 + POOL_QT, t0 + W) - 1;
  const int kb_last = qlast / BLK;

  bf16x8 bq[4][KS];
  int tq[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    tq[nt] = qt0 + 64 * wave + 16 * nt + l16;
    const bool ok = tq[nt] <= qlast;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      bq[nt][ks] = ok ? ld8(qp + ((size_t)(b * T + tq[nt]) * G + g) * DP + 32 * ks + 8 * q4) : zero8();
  }

  bf16x8 pre[CPT];
  auto gload = [&](int kb) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = threadIdx.x + 256 * u, r = c / (DP / 8), c8 = c % (DP / 8);
      pre[u] = ld8(kp + ((size_t)(b * T + kb * BLK + r) * G + g) * DP + 8 * c8);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = threadIdx.x + 256 * u, r = c / (DP / 8), c8 = c % (DP / 8);
      st8(&kbuf[buf][r * LDK + 8 * c8], pre[u]);
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kb = 0; kb <= kb_last; ++kb) {
    const int cur = kb & 1;
    if (kb < kb_last) gload(kb + 1);

    f32x4 acc[8][4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const bf16x8 a = ld8(&kbuf[cur][(16 * mt + l16) * LDK + 32 * ks + 8 * q4]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma16(a, bq[nt][ks], acc[mt][nt]);
      }

    // Keys after a query exist only in blocks that reach past this wave's first query.
    const bool need_mask = kb * BLK + BLK - 1 > qt0 + 64 * wave;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      float m = -INFINITY;
      const int lim = tq[nt] - kb * BLK;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float s = acc[mt][nt][e];
          if (need_mask && 16 * mt + 4 * q4 + e > lim) s = -INFINITY;
          m = fmaxf(m, s);
        }
      m = wave_max_xor_16_32(m);
      if (m == 0.0f) m = 0.0f;  // -0 and +0 rank equal
      if (q4 == 0) pbuf[(64 * wave + 16 * nt + l16) * (POOL_CHB + 1) + (kb % POOL_CHB)] = m;
    }
    if (kb < kb_last) lstore(cur ^ 1);
    __syncthreads();
    if ((kb % POOL_CHB) == POOL_CHB - 1 || kb == kb_last) {
      const int kb0 = kb - (kb % POOL_CHB);
      for (int i = threadIdx.x; i < POOL_QT * POOL_CHB; i += 256) {
        const int r = i / POOL_CHB, c = i % POOL_CHB, t = qt0 + r;
        if (kb0 + c <= kb && t <= qlast && kb0 + c <= t / BLK)
          pooled[((size_t)bg * W + (t - t0)) * N + kb0 + c] = pbuf[r * (POOL_CHB + 1) + c];
      }
      __syncthreads();
    }
  }
}

// Top-k of one pooled row per wavefront.  Scores become order-preserving u32
// keys held in registers (VPL per lane).  The k-th largest key is found by a
// three-digit radix select (11, 11 and 10 bits): each digit is histogrammed in
// LDS over the keys that match the digits found so far, and a wave scan from
// the top bin finds the bin where the count of larger keys reaches k.  Blocks
// above the k-th key are taken, then blocks equal to it lowest index first;
// a ballot pass writes the chosen block ids in ascending order, and the row
// tail is -1.
constexpr int TOPK_BINS = 2048;

template <int VPL>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ pooled, int32_t* __restrict__ idx,
                                              int T, int N, int K, int t0, int W, int rows) {
  __shared__ uint32_t hist_all[4][TOPK_BINS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t* hist = hist_all[wave];
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;  // whole wave exits: no block-level barrier below
  const int bg = row / W, tl = row % W, t = t0 + tl;
  const int nc = t / BLK + 1;
  const int nsel = min(K, nc);
  const float* pr = pooled + (size_t)row * N;

  uint32_t key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int col = i * 64 + lane;
    uint32_t kk = 0;
    if (col < nc) {
      float f = pr[col];
      if (f == 0.0f) f = 0.0f;  // -0 ranks equal to +0
      const uint32_t u = __float_as_uint(f);
      kk = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    }
    key[i] = kk;
  }

  uint32_t prefix = 0;
  int need = nsel;  // rank of the wanted key among keys matching prefix
  if constexpr (VPL <= 16) {
    // Short rows: build the k-th largest key bit by bit from the top; each
    // step is one ballot count per register of keys.
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = prefix | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (i * 64 < nc) cnt += __popcll(__ballot((i * 64 + lane < nc) && key[i] >= cand));
      if (cnt >= nsel) prefix = cand;
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
    for (int j = 0; j < per; ++j) {  // every lane walks the owner's bins (LDS broadcast)
      const uint32_t c = hist[otop - 1 - j];
      if (run + c >= (uint32_t)need) { bin = otop - 1 - j; break; }
      run += c;
    }
    need -= (int)run;
    prefix |= (uint32_t)bin << sh;
    bits = sh;
    __builtin_amdgcn_wave_barrier();
  }
  }
  const uint32_t kth = prefix;
  const int need_eq = need;  // equal keys to take, lowest block index first

  int32_t* out = idx + ((size_t)bg * T + t) * K;
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

hipError_t launch_proxy_pool(const Geo& g, const Win& w, const uint16_t* qp, const uint16_t* kp,
                             float* pooled, hipStream_t st) {
  dim3 grid((w.W + POOL_QT - 1) / POOL_QT, g.B * g.G), block(256);
  switch (g.DP) {
    case 32: k_proxy_pool<32><<<grid, block, 0, st>>>(qp, kp, pooled, g.T, g.G, g.N, w.t0, w.W); break;
    case 64: k_proxy_pool<64><<<grid, block, 0, st>>>(qp, kp, pooled, g.T, g.G, g.N, w.t0, w.W); break;
    case 128: k_proxy_pool<128><<<grid, block, 0, st>>>(qp, kp, pooled, g.T, g.G, g.N, w.t0, w.W); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_topk(const Geo& g, const Win& w, const float* pooled, int32_t* idx, hipStream_t st) {
  const int rows = g.B * g.G * w.W;
  dim3 grid((rows + 3) / 4), block(256);
  const int need = (g.N + 63) / 64;
#define MSA_TOPK_CASE(V)                                                                   \
  if (need <= V) {                                                                         \
    k_topk<V><<<grid, block, 0, st>>>(pooled, idx, g.T, g.N, g.K, w.t0, w.W, rows);       \
    return hipGetLastError();                                                              \
  }
  MSA_TOPK_CASE(1)
  MSA_TOPK_CASE(2)
  MSA_TOPK_CASE(4)
  MSA_TOPK_CASE(8)
  MSA_TOPK_CASE(16)
  MSA_TOPK_CASE(32)
  MSA_TOPK_CASE(64)
  MSA_TOPK_CASE(128)
#undef MSA_TOPK_CASE
  return hipErrorInvalidValue;
}

}  // namespace msa
