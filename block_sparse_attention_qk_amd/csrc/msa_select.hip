// Index Branch kernels for gfx950: proxy score + 128-key block max-pool, and
// the per-row top-k that fills the block-index cache.
//
// Method (pages: xcelit "Flash-MSA: Open-Source Sparse Attention Kernels
// Debut", section "How MSA works"; ai-beat "flash-msa-sparse-attention-
// training", paragraphs 1, 3, 4): one proxy head per KV group scores every
// query against every causal key, scores are max-pooled over 128-key blocks,
// and the top-k blocks per query are cached.  This is the only quadratic step.
#include <type_traits>

#include "msa_common.h"
#include "msa_internal.h"
#include "msa_topk.h"

namespace msa {

constexpr int POOL_WAVES = 8;  // waves per workgroup, 32 queries each
constexpr int POOL_QT = 32 * POOL_WAVES;  // queries per workgroup
constexpr int POOL_CHB = 8;    // pooled blocks collected in LDS per flush
constexpr int POOL_NBUF = 3;   // key-block ring in LDS (DMA two blocks ahead)

// Position of 16-byte chunk c of key row r in a proxy key tile of DP dims:
// rows of 2*DP bytes, 256/(2*DP) rows per LDS bank line; the XOR spreads 16
// consecutive rows over all banks for 16-byte operand reads.
template <int DP>
__device__ __forceinline__ int kswz(int r, int c) {
  constexpr int CPR = DP / 8, RPL = 128 / DP;
  return c ^ ((r / RPL) & (CPR - 1));
}

// Workgroup barrier that orders LDS only: this wave's LDS operations complete,
// then all waves meet.  Global-to-LDS copies still in flight are not waited
// for (the caller waits for exactly the ones it needs).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Pooled scores for the queries [t0, t0+W) of one (batch, group):
//   pooled[(bg*W + t - t0)*N + i] = max_{128i <= j <= min(128i+127, t)} qp[t].kp[j]
// for i <= t/128 (other entries are not written).
//
// Each wave owns 32 queries (one MFMA column tile) whose proxy rows stay in
// registers as B operands; small per-wave state keeps four waves per SIMD.  The product is taken transposed,
// S^T = Kp Qp^T on v_mfma_f32_32x32x16_bf16 with keys along M, so that a lane
// holds 16 keys of one query column per key tile: the block max is in-lane
// maxima and one cross-lane step.  Key blocks arrive in a three-deep LDS ring
// by global-to-LDS copies issued two blocks ahead; pooled values collect in a
// double-buffered LDS table and leave as 32-byte row segments.
template <int DP>
__global__ __launch_bounds__(64 * POOL_WAVES, DP <= 64 ? 4 : 2) void k_proxy_pool(const bf16raw* __restrict__ qp,
                                                       const bf16raw* __restrict__ kp,
                                                       float* __restrict__ pooled, int T, int G, int N,
                                                       int t0, int W) {
  constexpr int KS = DP / 16;          // k-steps of 16 over the proxy dim
  constexpr int CPR = DP / 8;          // 16-byte chunks per key row
  constexpr int NDMA = BLK * CPR / (64 * POOL_WAVES);  // 1 KiB copies per wave per key block
  constexpr int PST = POOL_CHB + 1;    // pooled table row stride (floats)
  // three ring slots as separate arrays: with the slot of every access known at
  // compile time, the copies into one slot are seen not to alias reads of another
  static_assert(POOL_NBUF == 3, "the ring is the three arrays below");
  __shared__ __attribute__((aligned(16))) bf16raw kslot0[BLK * DP];
  __shared__ __attribute__((aligned(16))) bf16raw kslot1[BLK * DP];
  __shared__ __attribute__((aligned(16))) bf16raw kslot2[BLK * DP];
  __shared__ float pbuf[2][POOL_QT * PST];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int bg = blockIdx.y, b = bg / G, g = bg % G;
  const int tile = gridDim.x - 1 - blockIdx.x;  // longest rows first
  const int qt0 = t0 + tile * POOL_QT;
  const int qlast = min(qt0 + POOL_QT, t0 + W) - 1;
  const int kb_last = qlast / BLK;

  // B operands: query column 32*wave + l32, proxy dims 16ks + 8h .. +7
  bf16x8 bq[KS];
  const int tq = qt0 + 32 * wave + l32;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    bq[ks] = tq <= qlast ? ld8(qp + ((size_t)(b * T + tq) * G + g) * DP + 16 * ks + 8 * h) : zero8();

  auto slot_ptr = [&](auto sl) -> bf16raw* {
    if constexpr (decltype(sl)::value == 0) return kslot0;
    else if constexpr (decltype(sl)::value == 1) return kslot1;
    else return kslot2;
  };
  // Copy of key block kb (clamped to the last one) into a ring slot.  Lane l of
  // copy u lands at slot byte 1024 (NDMA wave + u) + 16 l: key row r, physical
  // chunk p; it fetches the logical chunk p ^ swizzle(r).
  auto dma = [&](int kb, bf16raw* slot) {
    const int kbc = min(kb, kb_last);
#pragma unroll
    for (int u = 0; u < NDMA; ++u) {
      const int cidx = (NDMA * wave + u) * 64 + lane, r = cidx / CPR, pch = cidx % CPR;
      const bf16raw* src = kp + ((size_t)(b * T + kbc * BLK + r) * G + g) * DP + 8 * kswz<DP>(r, pch);
      __builtin_amdgcn_global_load_lds(src, slot + (NDMA * wave + u) * 512, 16, 0, 0);
    }
  };
  // Thread i writes block kb0 + i % 8 of the rows i / 8 + 64j.  Its row base is
  // formed here from an opaque copy of the thread index: held across the key
  // loop, it would be spilled, and reloading it would wait for the ring copies.
  auto flush = [&](int chunk) {  // pooled blocks [chunk*8, chunk*8+8) of the 256 queries
    constexpr int RSTEP = 64 * POOL_WAVES / POOL_CHB;
    const int kb0 = chunk * POOL_CHB;
    const float* pb = pbuf[chunk & 1];
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int c = tid % POOL_CHB, r0 = tid / POOL_CHB;
    if (kb0 + c <= kb_last) {
      float* dst = pooled + ((size_t)bg * W + (qt0 + r0 - t0)) * N + kb0 + c;
#pragma unroll
      for (int j = 0; j < POOL_QT / RSTEP; ++j) {
        const int r = r0 + RSTEP * j, t = qt0 + r;
        if (t <= qlast && kb0 + c <= t / BLK) dst[(size_t)RSTEP * j * N] = pb[r * PST + c];
      }
    }
  };

  // One key block: block kb is in slot SL, the copy of block kb+2 goes to slot (SL+2) % POOL_NBUF.
  auto step = [&](auto sl, int kb) {
    constexpr int SL = decltype(sl)::value;
    // a finished chunk of pooled values leaves first, so that its stores are
    // older than this step's copy and never held up by the wait below
    if (kb > 0 && kb % POOL_CHB == 0) flush(kb / POOL_CHB - 1);
    dma(kb + 2, slot_ptr(std::integral_constant<int, (SL + 2) % POOL_NBUF>{}));  // slot of block kb-1: finished

    const bf16raw* kc = slot_ptr(sl);
    const bool need_mask = kb * BLK + BLK - 1 > qt0 + 32 * wave;  // keys past some query of this wave
    const int lim = tq - kb * BLK;
    float mx = -INFINITY;
    // The causal mask is a separate compile-time path: blocks that no query of
    // the wave crosses (all but the last one or two) take only the maxima.
    auto tiles = [&](auto maskc) {
      constexpr bool MASK = decltype(maskc)::value;
      // The operands of tile mt+1 are read before the MFMAs of tile mt, into the
      // other of two register sets, so each tile's reads have a tile's work to land.
      bf16x8 ka[2][KS];
      auto rd = [&](int mt, int set) {
        const int r = 32 * mt + l32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) ka[set][ks] = ld8(&kc[r * DP + 8 * kswz<DP>(r, 2 * ks + h)]);
      };
      rd(0, 0);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {  // 32-key tiles (other waves of the SIMD cover the MFMA chain)
        if (mt + 1 < 4) rd(mt + 1, (mt + 1) & 1);
        f32x16 acc = zero16();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mfma32(ka[mt & 1][ks], bq[ks], acc);
        // lane holds query column l32 and keys 32mt + 8(e/4) + 4h + e%4
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float sv = acc[e];
          if constexpr (MASK) {
            if (32 * mt + 8 * (e >> 2) + 4 * h + (e & 3) > lim) sv = -INFINITY;
          }
          mx = fmaxf(mx, sv);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep later tiles' operand reads from piling up in registers
      }
    };
    if (need_mask)
      tiles(std::true_type{});
    else
      tiles(std::false_type{});
    {
      float m = fmaxf(mx, __shfl_xor(mx, 32));
      if (m == 0.0f) m = 0.0f;  // -0 and +0 rank equal
      if (h == 0) pbuf[(kb / POOL_CHB) & 1][(32 * wave + l32) * PST + (kb % POOL_CHB)] = m;
    }
    // block kb+1 must have landed: only this step's copy (NDMA per wave) may still be in flight
    __builtin_amdgcn_s_waitcnt(0x0f70 | NDMA);
    lds_barrier();
  };

  dma(0, kslot0);
  dma(1, kslot1);
  __builtin_amdgcn_s_waitcnt(0x0f70 | NDMA);  // vmcnt(NDMA): block 0 has landed (block 1 may be in flight)
  lds_barrier();
  // Three steps per pass without branches between them (a step past the last
  // block recomputes the last block; the flush drops its values).
  int kb = 0;
  for (; kb <= kb_last; kb += 3) {
    step(std::integral_constant<int, 0>{}, kb);
    step(std::integral_constant<int, 1>{}, kb + 1);
    step(std::integral_constant<int, 2>{}, kb + 2);
  }
  if ((kb - 1) / POOL_CHB == kb_last / POOL_CHB) flush(kb_last / POOL_CHB);  // unless a step already did
  // drain the ring copies still in flight before the workgroup ends
  __builtin_amdgcn_s_waitcnt(0x0f70);
}

template <int VPL>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ pooled, int32_t* __restrict__ idx,
                                              int T, int N, int K, int t0, int W, int rows) {
  __shared__ uint32_t hist_all[4][TOPK_ROW_LDS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;  // whole wave exits: no block-level barrier below
  const int bg = row / W, tl = row % W, t = t0 + tl;
  topk_row<VPL>(pooled + (size_t)row * N, t / BLK + 1, K, idx + ((size_t)bg * T + t) * K, hist_all[wave], lane);
}

// Long rows (more than 1024 blocks): one 512-thread workgroup per row, VPT
// keys per thread in columns i*512 + tid.  A wave per row would need 64 key
// registers or more per lane at these lengths (one wave per SIMD, spilled
// scalars); here each thread holds at most 16 keys and eight waves share the
// search for the k-th key: a histogram of 2048 bins spread linearly between
// the row's smallest and largest score, with the chosen bin's few keys ranked
// directly, else a radix select (11-bit digits below the row's common prefix,
// a workgroup scan from the top bin, an early stop when the chosen bin holds
// exactly the keys still needed).  The tie rule is the wave routine's: keys
// equal to the k-th are taken lowest block first.
constexpr int TKW_THREADS = 512;
constexpr int TKW_WAVES = TKW_THREADS / 64;
constexpr int TKW_CAND = 256;  // largest chosen linear bin ranked directly

template <int VPT>
__global__ __launch_bounds__(TKW_THREADS) void k_topk_wg(const float* __restrict__ pooled,
                                                         int32_t* __restrict__ idx, int T, int N, int K, int t0,
                                                         int W) {
  constexpr int PER = TOPK_BINS / TKW_THREADS;  // bins per thread in the scan of an 11-bit digit
  __shared__ uint32_t hist[TOPK_BINS];
  __shared__ uint32_t red[2][TKW_WAVES];
  __shared__ uint32_t wsum[TKW_WAVES];
  __shared__ int bc[3];
  __shared__ uint32_t cand[TKW_CAND];  // keys of the chosen linear bin
  __shared__ int ncand, kq[2];
  constexpr int NW = VPT * TKW_THREADS / 32;  // bitmap words per row
  __shared__ uint32_t gtw[NW], eqw[NW], wtot[TKW_WAVES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;  // the grid holds exactly the window's rows
  const int bg = row / W, t = t0 + row % W;
  const int nc = t / BLK + 1, nsel = min(K, nc);
  const float* pr = pooled + (size_t)row * N;
  int32_t* out = idx + ((size_t)bg * T + t) * K;

  // All loads in flight together: columns past the causal blocks read the
  // last causal score (nc >= 1) and are masked after.
  float sc[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) sc[i] = pr[min(i * TKW_THREADS + tid, nc - 1)];
  uint32_t key[VPT];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const bool valid = i * TKW_THREADS + tid < nc;
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
  for (int w = 0; w < TKW_WAVES; ++w) {
    kmin = min(kmin, red[0][w]);
    kmax = max(kmax, red[1][w]);
  }
  // The chosen bin of a histogram whose counts are in hist[0..nbins): the bin
  // holding the need-th largest key, counted from the top.  Writes bc = {bin,
  // rank of the wanted key inside the bin, the bin's count}; all threads read
  // bc after the second barrier (hist and wsum are next written after it).
  auto scan_bin = [&](int nbins, int need) {
    // thread tid owns the bins [top - PER, top) counted from the top bin down
    const int top = nbins - PER * tid;
    uint32_t c[PER], lsum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      c[j] = top - 1 - j >= 0 ? hist[top - 1 - j] : 0u;
      lsum += c[j];
    }
    uint32_t incl = lsum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < TKW_WAVES; ++w)
      if (w < wave) incl += wsum[w];
    const uint32_t excl = incl - lsum;
    if (excl < (uint32_t)need && (uint32_t)need <= incl) {  // exactly one thread
      uint32_t run = excl;
      int bin = top - 1;
      uint32_t cbin = 0;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        if (run + c[j] >= (uint32_t)need) {
          bin = top - 1 - j;
          cbin = c[j];
          break;
        }
        run += c[j];
      }
      bc[0] = bin;
      bc[1] = need - (int)run;
      bc[2] = (int)cbin;
    }
    __syncthreads();
  };

  uint32_t kth = 0u;
  int need_eq = 0;  // equal keys to take, lowest block index first
  bool done = false;
  if (nsel == nc) {  // every causal block is taken
    kth = kmin;
    need_eq = INT_MAX;
    done = true;
  } else {
    // First digit: 2048 bins spread linearly between the row's smallest and
    // largest score.  The bin is a non-decreasing function of the score, so
    // the wanted key lies in the chosen bin and every key of a higher bin is
    // larger.  Scores cluster far less in the upper tail than in the float
    // exponent, so the chosen bin holds a few keys, ranked directly.  Rows with
    // non-finite scores, equal extremes or a crowded bin take the radix path.
    const float fmin = key_score(kmin), fmax = key_score(kmax);
    const float span = fmax - fmin, scl = (float)TOPK_BINS / span;
    if (fmax > fmin && __builtin_isfinite(span) && __builtin_isfinite(scl) && scl > 0.f) {  // same in every thread
      int lb[VPT];
#pragma unroll
      for (int i = 0; i < VPT; ++i)
        lb[i] = i * TKW_THREADS + tid < nc ? min(TOPK_BINS - 1, (int)((sc[i] - fmin) * scl)) : -1;
      for (int j = tid; j < TOPK_BINS; j += TKW_THREADS) hist[j] = 0;
      if (tid == 0) {
        ncand = 0;
        kq[0] = (int)kmax;  // replaced below by the one key that satisfies the rank test
        kq[1] = 0;
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < VPT; ++i)
        if (lb[i] >= 0) atomicAdd(&hist[lb[i]], 1u);
      __syncthreads();
      scan_bin(TOPK_BINS, nsel);
      const int b = bc[0], needb = bc[1], cntb = bc[2];
      if (cntb <= TKW_CAND) {
#pragma unroll
        for (int i = 0; i < VPT; ++i)
          if (lb[i] == b) cand[atomicAdd(&ncand, 1)] = key[i];
        __syncthreads();
        if (tid < cntb) {  // the candidate whose key has needb - 1 larger ones and needb or more at least as large
          const uint32_t mine = cand[tid];
          int gt = 0, ge = 0;
          for (int j = 0; j < cntb; ++j) {
            const uint32_t o = cand[j];
            gt += o > mine;
            ge += o >= mine;
          }
          if (gt < needb && needb <= ge) {  // the same values from every candidate equal to it
            kq[0] = (int)mine;
            kq[1] = needb - gt;
          }
        }
        __syncthreads();
        kth = (uint32_t)kq[0];
        need_eq = kq[1];
        done = true;
      }
    }
  }
  if (!done) {
    // Radix select of the nsel-th largest key below the common prefix of kmin and kmax.
    const uint32_t diff = kmin ^ kmax;
    int bits = diff == 0u ? 0 : 32 - __builtin_clz(diff);
    uint32_t prefix = bits == 32 ? 0u : (kmax & ~((1u << bits) - 1u));
    int need = nsel;      // rank of the wanted key among the keys matching prefix
    bool all_eq = false;  // every key equal to the final prefix is taken
    while (bits > 0) {    // bits, prefix and need are the same in every thread
      const int width = bits < 11 ? bits : 11;
      const int sh = bits - width, nbins = 1 << width;
      const uint32_t hi_mask = bits == 32 ? 0u : ~((1u << bits) - 1u);
      for (int j = tid; j < nbins; j += TKW_THREADS) hist[j] = 0;
      __syncthreads();
  #pragma unroll
      for (int i = 0; i < VPT; ++i)
        if (i * TKW_THREADS + tid < nc && (key[i] & hi_mask) == prefix)
          atomicAdd(&hist[(key[i] >> sh) & (nbins - 1)], 1u);
      __syncthreads();
      scan_bin(nbins, need);
      prefix |= (uint32_t)bc[0] << sh;
      need = bc[1];
      bits = sh;
      // The chosen bin holds exactly the keys still needed: all of them are taken,
      // the lower digits cannot change that, and no other key ties with them.
      if (bc[2] == need) {
        all_eq = true;
        break;
      }
      // hist, wsum and bc are next written after two more barriers: no barrier here
    }
    kth = prefix;
    need_eq = all_eq ? INT_MAX : need;
  }

  // Ascending write-out from two bitmaps in LDS: word w holds columns
  // 32w .. 32w+31, above (gtw) or equal to (eqw) the k-th key.  Columns
  // i*512 + 64*wave + lane of one ballot are words 16i + 2*wave and the next.
  // Thread tid < NW then owns word tid: one workgroup scan of the packed
  // (above, equal) counts gives each word the chosen columns before it, since
  // equal keys are taken lowest column first and need_eq of them in all.
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const bool valid = i * TKW_THREADS + tid < nc;
    const unsigned long long mg = __ballot(valid && key[i] > kth);
    const unsigned long long me = __ballot(valid && key[i] == kth);
    if (lane == 0) {
      const int w = 16 * i + 2 * wave;
      gtw[w] = (uint32_t)mg;
      gtw[w + 1] = (uint32_t)(mg >> 32);
      eqw[w] = (uint32_t)me;
      eqw[w + 1] = (uint32_t)(me >> 32);
    }
  }
  __syncthreads();
  const uint32_t gw = tid < NW ? gtw[tid] : 0u, ew = tid < NW ? eqw[tid] : 0u;
  const uint32_t own = (uint32_t)__popc(gw) | ((uint32_t)__popc(ew) << 16);  // each count <= 8192
  uint32_t incl = own;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < TKW_WAVES; ++w)
    if (w < wave) incl += wtot[w];
  if (tid < NW) {
    const uint32_t excl = incl - own;
    const int gt_before = (int)(excl & 0xffffu), eq_before = (int)(excl >> 16);
    const int take = need_eq - eq_before;  // equal keys of this word still wanted
    uint32_t ek = 0u;
    if (take >= (int)__popc(ew)) {
      ek = ew;
    } else if (take > 0) {  // the lowest `take` set bits
      uint32_t r = ew;
      for (int j = 0; j < take; ++j) {
        ek |= r & (0u - r);
        r &= r - 1u;
      }
    }
    uint32_t ch = gw | ek;
    int pos = gt_before + min(eq_before, need_eq);
    while (ch != 0u) {
      if ((unsigned)pos < (unsigned)nsel) out[pos] = 32 * tid + __ffs(ch) - 1;
      ++pos;
      ch &= ch - 1u;
    }
  }
  for (int p = nsel + tid; p < K; p += TKW_THREADS) out[p] = -1;
}

hipError_t launch_proxy_pool(const Geo& g, const Win& w, const uint16_t* qp, const uint16_t* kp,
                             float* pooled, hipStream_t st) {
  dim3 grid((w.W + POOL_QT - 1) / POOL_QT, g.B * g.G), block(64 * POOL_WAVES);
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
#undef MSA_TOPK_CASE
  // rows of more than 1024 blocks: one workgroup per row
  const int vpt = (g.N + TKW_THREADS - 1) / TKW_THREADS;
#define MSA_TOPK_WG_CASE(V)                                                                 \
  if (vpt <= V) {                                                                           \
    k_topk_wg<V><<<dim3(rows), dim3(TKW_THREADS), 0, st>>>(pooled, idx, g.T, g.N, g.K, w.t0, w.W); \
    return hipGetLastError();                                                               \
  }
  MSA_TOPK_WG_CASE(4)
  MSA_TOPK_WG_CASE(8)
  MSA_TOPK_WG_CASE(16)
#undef MSA_TOPK_WG_CASE
  return hipErrorInvalidValue;
}

}  // namespace msa
