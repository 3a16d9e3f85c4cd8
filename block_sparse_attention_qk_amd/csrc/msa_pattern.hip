// Fixed window/dilation block pattern, optionally united with a given cache
// (keelcrux "Flash-MSA: Train on a million tokens without breaking the compute
// bank", section "Under the hood": the block pattern is configurable by window
// size and dilation).  The pages give no definition; the reading, stated with
// the C ABI, is: the `window` most recent causal blocks, every causal block
// below the window whose index is a multiple of `dilation`, and the causal
// entries of an input cache row, listed once each in ascending order.
#include "msa_common.h"
#include "msa_internal.h"

namespace msa {

constexpr int PAT_MAXN = 1 << 13;  // blocks per row at the longest supported T (2^20 tokens)

// One row per wavefront.  The input row's blocks below the window are marked
// in an LDS bitmap; a ballot pass over the causal blocks then writes the
// selected block ids in ascending order.
__global__ __launch_bounds__(256) void k_pattern(const int32_t* __restrict__ idx_in, int k_in,
                                                 int32_t* __restrict__ idx_out, int K, int T, int window,
                                                 int dilation, long long rows) {
  __shared__ uint32_t bits[4][PAT_MAXN / 32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * 4 + wave;
  if (row >= rows) return;  // whole wave exits; no workgroup barrier below
  const int t = (int)(row % T);
  const int nc = t / BLK + 1, lo = max(0, nc - window);
  uint32_t* bm = bits[wave];
  if (idx_in != nullptr) {
    const int nw = (lo + 31) / 32;
    for (int i = lane; i < nw; i += 64) bm[i] = 0u;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // cleared before any lane marks
    const int32_t* ir = idx_in + row * k_in;
    for (int e = lane; e < k_in; e += 64) {
      const int b = ir[e];
      if (b >= 0 && b < lo) atomicOr(&bm[b >> 5], 1u << (b & 31));
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // every mark lands before the reads
  }
  int32_t* out = idx_out + row * K;
  const unsigned long long lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int n = 0;
  for (int b0 = 0; b0 < nc; b0 += 64) {
    const int b = b0 + lane;
    bool sel = false;
    if (b < nc) {
      sel = b >= lo || (dilation > 0 && b % dilation == 0);
      if (!sel && idx_in != nullptr) sel = (bm[b >> 5] >> (b & 31)) & 1u;
    }
    const unsigned long long m = __ballot(sel);
    if (sel) out[n + __popcll(m & lt)] = b;
    n += __popcll(m);
  }
  for (int p = n + lane; p < K; p += 64) out[p] = -1;
}

hipError_t launch_pattern(const int32_t* idx_in, int k_in, int32_t* idx_out, int K, int B, int G, int T,
                          int window, int dilation, hipStream_t st) {
  const long long rows = (long long)B * G * T;
  const long long blocks = (rows + 3) / 4;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  k_pattern<<<dim3((unsigned)blocks), 256, 0, st>>>(idx_in, k_in, idx_out, K, T, window, dilation, rows);
  return hipGetLastError();
}

}  // namespace msa
