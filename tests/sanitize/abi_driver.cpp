// Calls every libmsa entry point with arguments that its host-side checks
// reject (so nothing reaches the GPU), plus the size queries over a sweep of
// shapes, so that a build of the host code with AddressSanitizer and
// UndefinedBehaviorSanitizer can watch the validation, layout and window
// arithmetic (test infrastructure: built and run by tests/test_sanitizers.py,
// no GPU needed).  Exit status 0 when every call returns the expected code.
#include <cstdint>
#include <cstdio>

#include "msa.h"

#define EXPECT(call, code)                                                                          \
  do {                                                                                              \
    const int rc_ = (int)(call);                                                                    \
    if (rc_ != (int)(code)) {                                                                       \
      std::fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, rc_,  \
                   (int)(code));                                                                    \
      return 1;                                                                                     \
    }                                                                                               \
  } while (0)

extern "C" int abi_enum_range_checks(void);  // abi_enum.c: out-of-range enum arguments

int main() {
  void* P = reinterpret_cast<void*>(uintptr_t{4096});
  void* Q = reinterpret_cast<void*>(uintptr_t{4096 + 8});  // misaligned
  auto b = [](void* p) { return static_cast<msa_bf16*>(p); };
  auto i = [](void* p) { return static_cast<int32_t*>(p); };
  auto f = [](void* p) { return static_cast<float*>(p); };

  // size queries over shapes, ops and the window search
  const int Ts[] = {128, 384, 1024, 131072, 1 << 20};
  const int ks[] = {1, 4, 32, 288, 1024};
  size_t total = 0;
  for (int T : Ts)
    for (int k : ks)
      for (int op = MSA_OP_SELECT; op <= MSA_OP_FWD_BWD; ++op) {
        msa_dims d = {1, T, 16, 2, 128, 64, k, 0.f};
        total += msa_workspace_bytes(&d, (msa_op)op) + msa_workspace_min_bytes(&d, (msa_op)op);
      }
  if (total == 0) return 1;

  EXPECT(abi_enum_range_checks(), 0);
  msa_dims d = {1, 1024, 8, 2, 128, 64, 4, 0.f};
  const size_t ws = msa_workspace_bytes(&d, MSA_OP_BWD);
  msa_dims bad_T = d, bad_R = d, bad_hd = d, nan_scale = d;
  bad_T.T = 1000;
  bad_R.H = 6;
  bad_hd.d = 96;
  nan_scale.scale = 0.f / 0.f;
  EXPECT(msa_proxy_select(nullptr, b(P), b(P), i(P), P, ws, nullptr), MSA_ERR_NULL);
  EXPECT(msa_proxy_select(&bad_T, b(P), b(P), i(P), P, ws, nullptr), MSA_ERR_SHAPE);
  EXPECT(msa_proxy_select(&d, b(Q), b(P), i(P), P, ws, nullptr), MSA_ERR_ALIGN);
  EXPECT(msa_proxy_select(&d, b(P), b(P), i(P), P, 16, nullptr), MSA_ERR_WORKSPACE);
  EXPECT(msa_fwd(&d, b(P), b(P), b(P), i(P), b(P), f(P), P, 0, nullptr), MSA_ERR_WORKSPACE);
  EXPECT(msa_fwd(&bad_R, b(P), b(P), b(P), i(P), b(P), f(P), P, ws, nullptr), MSA_ERR_UNSUPPORTED);
  EXPECT(msa_fwd(&nan_scale, b(P), b(P), b(P), i(P), b(P), f(P), P, ws, nullptr), MSA_ERR_SHAPE);
  EXPECT(msa_fwd(&d, b(P), nullptr, b(P), i(P), b(P), f(P), P, ws, nullptr), MSA_ERR_NULL);
  EXPECT(msa_bwd(&bad_hd, b(P), b(P), b(P), b(P), b(P), f(P), i(P), b(P), b(P), b(P), P, ws, nullptr),
         MSA_ERR_UNSUPPORTED);
  EXPECT(msa_bwd(&d, b(P), b(P), b(P), b(P), b(P), f(P), i(P), b(P), b(P), b(Q), P, ws, nullptr), MSA_ERR_ALIGN);
  EXPECT(msa_bwd(&d, b(P), b(P), b(P), b(P), b(P), f(P), i(P), b(P), b(P), b(P), P, 100, nullptr),
         MSA_ERR_WORKSPACE);
  EXPECT(msa_fwd_bwd(&d, b(P), b(P), b(P), b(P), i(P), b(P), f(P), b(P), b(P), b(P), P, 100, nullptr),
         MSA_ERR_WORKSPACE);
  EXPECT(msa_pattern_select(&d, -1, 0, nullptr, 0, i(P), nullptr), MSA_ERR_SHAPE);
  EXPECT(msa_pattern_select(&d, 8, 64, nullptr, 0, i(P), nullptr), MSA_ERR_SHAPE);  // rows wider than topk 4
  EXPECT(msa_decode_select(&d, b(P), b(P), i(P), i(P), P, 0, nullptr), MSA_ERR_WORKSPACE);
  EXPECT(msa_decode_fwd(&d, b(P), b(P), b(P), i(P), i(P), b(P), f(P), nullptr, 0, nullptr), MSA_ERR_NULL);
  EXPECT(msa_decode_fwd_static(&d, b(P), b(P), b(Q), i(P), i(P), b(P), f(P), nullptr), MSA_ERR_ALIGN);
  msa_dims big = {64, 256, 32, 4, 128, 64, 32, 0.f};
  EXPECT(msa_decode_fwd_static(&big, b(P), b(P), b(P), i(P), i(P), b(P), f(P), nullptr), MSA_ERR_SCRATCH);
  for (int s = MSA_OK; s <= MSA_ERR_SCRATCH; ++s)
    if (msa_status_str((msa_status)s) == nullptr) return 1;
  double ms[MSA_K_COUNT];
  int32_t n[MSA_K_COUNT];
  EXPECT(msa_timing_read(ms, n, MSA_K_COUNT), MSA_OK);  // nothing recorded on this thread
  msa_timing_enable(0);
  std::printf("abi driver ok (%s)\n", msa_version());
  return 0;
}
