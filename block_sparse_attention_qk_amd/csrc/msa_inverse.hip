// Inverse of the block-index cache for one window of tokens: for every
// (batch, group, block) the list of (token, slot) pairs that selected it, plus
// the work items the KV-stationary Main Branch kernels walk.
//
// The cache is the block-index table the Index Branch writes (xcelit page,
// "How MSA works": everything downstream reads the cached sparse blocks).  Its
// inverse lets the Main Branch keep one K/V block in LDS and stream the queries
// that read it.  Built as a counting sort: per-chunk block histograms in LDS,
// a column scan over chunks, a scan over blocks, then a scatter.
#include "msa_common.h"
#include "msa_internal.h"

namespace msa {

constexpr int INV_THREADS = 512;  // threads per counting-sort workgroup
constexpr int INV_UNROLL = 8;     // cache entries each thread loads before its LDS atomics

// counts[bg][chunk][blk] = number of pairs of the chunk's tokens that picked blk.
// Entries outside 0..t/128 are ignored.
__global__ __launch_bounds__(INV_THREADS) void k_inv_count(const int32_t* __restrict__ idx,
                                                           int32_t* __restrict__ counts, int T, int N, int K,
                                                           int t0, int W, int nchunk) {
  extern __shared__ int32_t hist[];
  const int chunk = blockIdx.x, bg = blockIdx.y;
  for (int i = threadIdx.x; i < N; i += INV_THREADS) hist[i] = 0;
  __syncthreads();
  const int tl0 = chunk * INV_CHUNK, n = min(INV_CHUNK, W - tl0) * K;
  const int32_t* rows = idx + ((size_t)bg * T + t0 + tl0) * K;
  for (int e0 = threadIdx.x; e0 < n; e0 += INV_THREADS * INV_UNROLL) {
    int blk[INV_UNROLL];
#pragma unroll
    for (int u = 0; u < INV_UNROLL; ++u) {
      const int e = e0 + u * INV_THREADS;
      blk[u] = e < n ? rows[e] : -1;
    }
#pragma unroll
    for (int u = 0; u < INV_UNROLL; ++u) {
      const int e = e0 + u * INV_THREADS;
      if (blk[u] >= 0 && blk[u] <= (t0 + tl0 + e / K) / BLK) atomicAdd(&hist[blk[u]], 1);
    }
  }
  __syncthreads();
  int32_t* out = counts + ((size_t)bg * nchunk + chunk) * N;
  for (int i = threadIdx.x; i < N; i += INV_THREADS) out[i] = hist[i];
}

// In place: counts[bg][c][blk] <- sum over chunks before c; len[bg][blk] = total.
// Eight chunks' counts are loaded before their prefixes are stored.
__global__ __launch_bounds__(256) void k_inv_colscan(int32_t* __restrict__ counts, int32_t* __restrict__ len,
                                                     int N, int nchunk) {
  const int bg = blockIdx.y, blk = blockIdx.x * 256 + threadIdx.x;
  if (blk >= N) return;
  int32_t* col = counts + (size_t)bg * nchunk * N + blk;
  int run = 0;
  for (int c0 = 0; c0 < nchunk; c0 += INV_UNROLL) {
    int v[INV_UNROLL];
#pragma unroll
    for (int u = 0; u < INV_UNROLL; ++u) v[u] = c0 + u < nchunk ? col[(size_t)(c0 + u) * N] : 0;
#pragma unroll
    for (int u = 0; u < INV_UNROLL; ++u) {
      if (c0 + u < nchunk) col[(size_t)(c0 + u) * N] = run;
      run += v[u];
    }
  }
  len[(size_t)bg * N + blk] = run;
}

// One workgroup per (batch, group): exclusive scan of list lengths -> base,
// and the work items {block, start, len, flags} that cut each list into pieces
// of at most item_tokens pairs, in block order (flags: ITEM_SPLIT when a
// block's list spans several items, ITEM_DIAG on a block's first item).
__global__ __launch_bounds__(1024) void k_inv_blockscan(const int32_t* __restrict__ len, int32_t* __restrict__ base,
                                                        int4* __restrict__ items, int32_t* __restrict__ item_count,
                                                        int N, int max_items, int item_tokens) {
  __shared__ int s_a[1024], s_b[1024];
  const int bg = blockIdx.x, tid = threadIdx.x;
  const int per = (N + 1023) / 1024, b0 = tid * per;
  const int32_t* L = len + (size_t)bg * N;
  int sl = 0, si = 0;
  for (int i = 0; i < per; ++i) {
    const int blk = b0 + i;
    if (blk < N) {
      const int l = L[blk];
      sl += l;
      si += (l + item_tokens - 1) / item_tokens;
    }
  }
  s_a[tid] = sl;
  s_b[tid] = si;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int a = tid >= off ? s_a[tid - off] : 0, b = tid >= off ? s_b[tid - off] : 0;
    __syncthreads();
    s_a[tid] += a;
    s_b[tid] += b;
    __syncthreads();
  }
  int run_l = s_a[tid] - sl, run_i = s_b[tid] - si;
  if (tid == 1023) item_count[bg] = s_b[1023];
  int4* it = items + (size_t)bg * max_items;
  for (int i = 0; i < per; ++i) {
    const int blk = b0 + i;
    if (blk >= N) break;
    const int l = L[blk];
    base[(size_t)bg * N + blk] = run_l;
    const int split = l > item_tokens ? ITEM_SPLIT : 0;
    for (int s = 0; s < l; s += item_tokens)
      it[run_i++] = make_int4(blk, run_l + s, min(item_tokens, l - s), split | (s == 0 ? ITEM_DIAG : 0));
    run_l += l;
  }
}

// list[bg][pos] = (t - t0) << LIST_SLOT_BITS | slot, grouped by block.
__global__ __launch_bounds__(INV_THREADS) void k_inv_scatter(const int32_t* __restrict__ idx,
                                                             const int32_t* __restrict__ counts,
                                                             const int32_t* __restrict__ base,
                                                             int32_t* __restrict__ list, int T, int N, int K, int t0,
                                                             int W, int nchunk) {
  extern __shared__ int32_t cur[];
  const int chunk = blockIdx.x, bg = blockIdx.y;
  const int32_t* cc = counts + ((size_t)bg * nchunk + chunk) * N;
  const int32_t* bs = base + (size_t)bg * N;
  for (int i = threadIdx.x; i < N; i += INV_THREADS) cur[i] = bs[i] + cc[i];
  __syncthreads();
  const int tl0 = chunk * INV_CHUNK, n = min(INV_CHUNK, W - tl0) * K;
  const int32_t* rows = idx + ((size_t)bg * T + t0 + tl0) * K;
  int32_t* out = list + (size_t)bg * W * K;
  for (int e0 = threadIdx.x; e0 < n; e0 += INV_THREADS * INV_UNROLL) {
    int blk[INV_UNROLL];
#pragma unroll
    for (int u = 0; u < INV_UNROLL; ++u) {
      const int e = e0 + u * INV_THREADS;
      blk[u] = e < n ? rows[e] : -1;
    }
#pragma unroll
    for (int u = 0; u < INV_UNROLL; ++u) {
      const int e = e0 + u * INV_THREADS;
      const int tl = tl0 + e / K;
      if (blk[u] >= 0 && blk[u] <= (t0 + tl) / BLK) {
        const int pos = atomicAdd(&cur[blk[u]], 1);
        out[pos] = (tl << LIST_SLOT_BITS) | (e - (tl - tl0) * K);
      }
    }
  }
}

// Check of a block-index cache, one wave per row (b, g, t): every entry is -1
// or a causal block 0..t/128, no block appears twice (an LDS bitmap of the
// row's blocks, N <= 8192 bits), and at least one entry is a block.  A failing
// row writes 1 to flag[0]; flag[0] must be 0 before the launch.
constexpr int CHK_WAVES = 4;
constexpr int CHK_WORDS = 8192 / 32;

__global__ __launch_bounds__(64 * CHK_WAVES) void k_check_idx(const int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ flag, int T, int K,
                                                             long long rows) {
  __shared__ uint32_t seen[CHK_WAVES][CHK_WORDS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * CHK_WAVES + wave;
  if (row >= rows) return;  // whole wave: no workgroup barrier below
  const int last = (int)(row % T) / BLK;
  uint32_t* bm = seen[wave];
  for (int i = lane; i <= last / 32; i += 64) bm[i] = 0;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's clears land before its bitmap updates
  const int32_t* r = idx + row * K;
  bool bad = false, any = false;
  for (int p = lane; p < K; p += 64) {
    const int e = r[p];
    if (e == -1) continue;
    if (e < 0 || e > last) {
      bad = true;
      continue;
    }
    any = true;
    const uint32_t bit = 1u << (e & 31);
    if (atomicOr(&bm[e >> 5], bit) & bit) bad = true;
  }
  const bool row_any = __ballot(any) != 0ull;
  if (bad || (lane == 0 && !row_any)) flag[0] = 1;
}

hipError_t launch_check_idx(const Geo& g, const int32_t* idx, int32_t* flag, hipStream_t st) {
  if (g.N > 8192) return hipErrorInvalidValue;
  const long long rows = (long long)g.B * g.G * g.T;
  k_check_idx<<<(unsigned)((rows + CHK_WAVES - 1) / CHK_WAVES), 64 * CHK_WAVES, 0, st>>>(idx, flag, g.T, g.K, rows);
  return hipGetLastError();
}

// Dispatch order of a (batch, group)'s work items: by the middle token of
// their run (the mean of its first and last token; a counting sort into
// ORD_BINS token buckets), so that the items running at one time gather query
// rows from a narrow token range.  Items of one bucket keep no particular
// order among themselves.
constexpr int ORD_THREADS = 1024, ORD_BINS = 1024;
__global__ __launch_bounds__(ORD_THREADS) void k_item_order(const int4* __restrict__ items,
                                                           const int32_t* __restrict__ item_count,
                                                           const int32_t* __restrict__ list, int32_t* __restrict__ order,
                                                           int max_items, int K, int W) {
  __shared__ int cnt[ORD_BINS];
  __shared__ int wsum[ORD_THREADS / 64];
  const int bg = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = item_count[bg];
  const int4* it = items + (size_t)bg * max_items;
  const int32_t* lst = list + (size_t)bg * W * K;
  int32_t* ord = order + (size_t)bg * max_items;
  int shift = 0;
  while ((W >> shift) > ORD_BINS) ++shift;
  cnt[tid] = 0;
  __syncthreads();
  // an item holds at least one pair, so its last entry is start + len - 1
  auto bucket = [&](int i) {
    const int4 e = it[i];
    const int mid = ((lst[e.y] >> LIST_SLOT_BITS) + (lst[e.y + e.z - 1] >> LIST_SLOT_BITS)) / 2;
    return min(ORD_BINS - 1, mid >> shift);
  };
  for (int i = tid; i < n; i += ORD_THREADS) atomicAdd(&cnt[bucket(i)], 1);
  __syncthreads();
  const int own = cnt[tid];
  int incl = own;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  for (int w = 0; w < wave; ++w) incl += wsum[w];
  cnt[tid] = incl - own;  // first position of bucket tid
  __syncthreads();
  for (int i = tid; i < n; i += ORD_THREADS)
    ord[atomicAdd(&cnt[bucket(i)], 1)] = i;
}

hipError_t launch_item_order(const Geo& g, const Win& w, const InvBufs& ib, hipStream_t st) {
  k_item_order<<<g.B * g.G, ORD_THREADS, 0, st>>>(ib.items, ib.item_count, ib.list, ib.order, ib.max_items, g.K, w.W);
  return hipGetLastError();
}

int inv_max_items(const Geo& g, int W, int item_tokens) {
  const long long pairs = (long long)W * g.K;
  long long m = g.N + pairs / item_tokens + 1;
  if (m > pairs + g.N) m = pairs + g.N;
  return (int)m;
}

hipError_t launch_inverse(const Geo& g, const Win& w, const int32_t* idx, const InvBufs& ib, int item_tokens,
                          hipStream_t st) {
  const int BG = g.B * g.G;
  const int nchunk = (w.W + INV_CHUNK - 1) / INV_CHUNK;
  const size_t lds = (size_t)g.N * sizeof(int32_t);
  k_inv_count<<<dim3(nchunk, BG), INV_THREADS, lds, st>>>(idx, ib.counts, g.T, g.N, g.K, w.t0, w.W, nchunk);
  k_inv_colscan<<<dim3((g.N + 255) / 256, BG), 256, 0, st>>>(ib.counts, ib.len, g.N, nchunk);
  k_inv_blockscan<<<BG, 1024, 0, st>>>(ib.len, ib.base, ib.items, ib.item_count, g.N, ib.max_items, item_tokens);
  k_inv_scatter<<<dim3(nchunk, BG), INV_THREADS, lds, st>>>(idx, ib.counts, ib.base, ib.list, g.T, g.N, g.K, w.t0, w.W,
                                                     nchunk);
  return hipGetLastError();
}

hipError_t launch_inverse_items(const Geo& g, const InvBufs& ib, int item_tokens, hipStream_t st) {
  k_inv_blockscan<<<g.B * g.G, 1024, 0, st>>>(ib.len, ib.base, ib.items, ib.item_count, g.N, ib.max_items,
                                               item_tokens);
  return hipGetLastError();
}

}  // namespace msa
