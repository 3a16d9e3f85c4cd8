// Host-side launchers of the gfx950 kernels (internal to libmsa).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

// Geometry shared by every kernel of one call.
struct Geo {
  int B, T, H, G, D, DP, K;  // K = topk
  int R, N;                  // R = H / G, N = T / 128
  float scale;               // softmax scale
};

// One window of tokens [t0, t0 + W).
struct Win {
  int t0, W;
};

constexpr int INV_CHUNK = 256;  // tokens per counting-sort chunk
constexpr int FWD_ITEM_TOKENS = 512;  // tokens per forward work item (list chunk)
// Backward items hold at most this many pairs: a block picked by more tokens
// (early blocks, or a fixed pattern's far blocks that every query reads) is cut
// into several items that run in parallel and add their dK/dV atomically.
constexpr int BWD_ITEM_TOKENS = 1024;

// Pair-list entries hold (t - t0) << LIST_SLOT_BITS | slot: the token offset
// in the window and the cache slot (topk <= 1024, windows <= 2^20 tokens).
constexpr int LIST_SLOT_BITS = 10;
// Work item flags (.w of {block, start, len, flags}).
constexpr int ITEM_SPLIT = 1;  // the block's list is cut into several items
constexpr int ITEM_DIAG = 2;   // the block's first item: the only one that can hold the block's own tokens
// The block's own tokens sit in the first counting-sort chunk of its list, so
// they all fall into its first item as long as an item holds a whole chunk.
static_assert(FWD_ITEM_TOKENS >= INV_CHUNK && BWD_ITEM_TOKENS >= INV_CHUNK, "items must hold a whole chunk");

// ---- Index Branch
hipError_t launch_proxy_pool(const Geo& g, const Win& w, const uint16_t* qp, const uint16_t* kp,
                             float* pooled, hipStream_t st);
hipError_t launch_topk(const Geo& g, const Win& w, const float* pooled, int32_t* idx, hipStream_t st);

// ---- Inverse (block -> selecting pairs) index for one window
struct InvBufs {
  int32_t* counts;      // [BG][nchunk][N]
  int32_t* base;        // [BG][N]   list start of each block
  int32_t* len;         // [BG][N]   list length of each block
  int4* items;          // [BG][max_items]  {block, start, len, ITEM_* flags}
  int32_t* item_count;  // [BG]
  int32_t* list;        // [BG][W * K]  entries (t - t0) << LIST_SLOT_BITS | slot
  int32_t* order;       // [BG][max_items]  dispatch order of the items (by middle token)
  int max_items;
};
int inv_max_items(const Geo& g, int W, int item_tokens);
hipError_t launch_inverse(const Geo& g, const Win& w, const int32_t* idx, const InvBufs& ib,
                          int item_tokens, hipStream_t st);
// Device check of a block-index cache: flag[0] (zero before the launch) becomes
// 1 if a row has an entry that is neither -1 nor a causal block, a repeated
// block, or no block at all.
hipError_t launch_check_idx(const Geo& g, const int32_t* idx, int32_t* flag, hipStream_t st);
// Dispatch order of ib's items (ib.order): by the middle token of each item's run.
hipError_t launch_item_order(const Geo& g, const Win& w, const InvBufs& ib, hipStream_t st);
// Work items {block, start, len, split} of the inverse index already built in
// `ib` (counts/len/base/list), cut at another item size into ib's items buffer.
hipError_t launch_inverse_items(const Geo& g, const InvBufs& ib, int item_tokens, hipStream_t st);

// ---- Main Branch
hipError_t launch_fwd_partials(const Geo& g, const Win& w, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const InvBufs& ib, uint16_t* part_o,
                               float* part_lse, hipStream_t st);
// dout/Dd non-null: also D = rowsum(dout * o) into Dd [B, T, H] (merged forward/backward)
hipError_t launch_fwd_combine(const Geo& g, const Win& w, const int32_t* idx, const uint16_t* part_o,
                              const float* part_lse, uint16_t* o, float* lse, const uint16_t* dout, float* Dd,
                              hipStream_t st);

hipError_t launch_bwd_dot(const Geo& g, const uint16_t* o, const uint16_t* dout, float* Dd, hipStream_t st);
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t st);
hipError_t launch_bwd_partials(const Geo& g, const Win& w, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const uint16_t* dout, const float* lse,
                               const float* Dd, const InvBufs& ib, uint16_t* dq_part,
                               float* dk_acc, float* dv_acc, hipStream_t st);
hipError_t launch_dq_combine(const Geo& g, const Win& w, const int32_t* idx, const uint16_t* dq_part,
                             uint16_t* dq, hipStream_t st);
hipError_t launch_cvt_bf16(const float* src, uint16_t* dst, size_t n, hipStream_t st);
hipError_t launch_pattern(const int32_t* idx_in, int k_in, int32_t* idx_out, int K, int B, int G, int T,
                          int window, int dilation, hipStream_t st);

// ---- Decode step (one new query per sequence; caches [B, T, G, *])
hipError_t launch_dec_pool(const Geo& g, const uint16_t* qp, const uint16_t* kp, const int32_t* len, float* pooled,
                           hipStream_t st);
hipError_t launch_dec_topk(const Geo& g, const float* pooled, const int32_t* len, int32_t* idx, hipStream_t st);
hipError_t launch_dec_attn(const Geo& g, const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* len,
                           const int32_t* idx, float* part_o, float* part_lse, hipStream_t st);
hipError_t launch_dec_combine(const Geo& g, const float* part_o, const float* part_lse, const int32_t* idx,
                              const int32_t* len, uint16_t* o, float* lse, hipStream_t st);

}  // namespace msa
