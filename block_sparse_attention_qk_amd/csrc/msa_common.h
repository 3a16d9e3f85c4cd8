// Device-side helpers shared by the gfx950 kernels of the MSA hot path.
//
// Matrix-core conventions (v_mfma_f32_16x16x32_bf16, one 64-lane wavefront):
//   A operand (16 x 32): lane l holds row (l % 16) and 8 consecutive K slots
//                        of slot group (l / 16).
//   B operand (32 x 16): lane l holds column (l % 16), same 8 K slots.
//   C/D       (16 x 16): lane l holds column (l % 16), rows 4*(l/16) + e, e<4.
// The sum over K pairs A's slot (group, e) with B's slot (group, e), so any
// assignment of K indices to slots works as long as A and B agree on it.
//
// Two 16x16 C tiles that are stacked along M (rows 0-15 and 16-31) can be fed
// straight into a following product that reduces over that M index: lane l
// holds the C values of rows {4q..4q+3} of the first tile and {4q..4q+3} of the
// second (q = l/16), which becomes K slots e = 0..3 and e = 4..7 of group q.
// kperm() gives the storage position of a K index under that slot order, so
// the other operand can be laid out in LDS to match and read with one 16-byte
// load per lane.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int BLK = 128;  // keys per KV block

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef uint16_t bf16raw;

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short i16x4;

// v_mfma_f32_32x32x16_bf16.  A (32 x 16): lane l holds row l%32, K slots
// 8*(l/32)+e.  B (16 x 32): lane l holds column l%32, same K slots.
// C (32 x 32): lane l holds column l%32, rows 8*(e/4) + 4*(l/32) + e%4 for
// e = 0..15.  Elements e = 8s..8s+7 of a C tile are therefore K slots e-8s of
// a following product that reduces over the C tile's rows, K step s, with
// slot (h = l/32, e') <-> row 16s + 8*(e'/4) + 4h + e'%4.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane
// j receives element j%4 of the 8-byte rows read by lanes 4e + j/4, e = 0..3.
// If lane i of the group points at row (r0 + i/4), columns (n0 + 4*(i%4)) of a
// row-major bf16 matrix, lane j receives M[r0 + e][n0 + j] for e = 0..3: four
// consecutive rows of its own column.
__device__ __forceinline__ uint2 lds_tr4(const void* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }


// Position of K index i (0..31) inside a 32-wide K step when the operand was
// produced from two stacked C tiles (see above).
__host__ __device__ constexpr int kperm(int i) {
  return 8 * ((i & 15) >> 2) + ((i >> 4) << 2) + (i & 3);
}


__device__ __forceinline__ bf16x8 ld8(const void* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void st8(void* p, const bf16x8& v) { *reinterpret_cast<bf16x8*>(p) = v; }

__device__ __forceinline__ uint4 ld16u(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16u(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }
// 16-byte store marked non-temporal: data written once and read back much
// later (the per-pair partials) streams past the caches instead of evicting
// rows that are still being re-read.
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
__device__ __forceinline__ void st16nt(void* p, const uint4& v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}
// 16-byte load marked non-temporal, for streams read exactly once (the
// partials in the combines, the proxy-key cache in decode): their lines are
// not kept, so they do not displace data that is read again.
__device__ __forceinline__ uint4 ld16nt(const void* p) {
  const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ bf16x8 as_bf8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

// Transposing two 8-element rows a, b (as 4 words each) into 8 words of
// (a[i], b[i]) pairs: word 2m is (a[2m], b[2m]), word 2m+1 is (a[2m+1], b[2m+1]).
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }
__device__ __forceinline__ uint32_t word_of(const uint4& v, int m) {
  return m == 0 ? v.x : m == 1 ? v.y : m == 2 ? v.z : v.w;
}

__device__ __forceinline__ float bf2f(bf16raw x) { return __uint_as_float(((uint32_t)x) << 16); }
__device__ __forceinline__ bf16raw f2bf(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(bf16raw, b);
}

__device__ __forceinline__ bf16x8 zero8() { return as_bf8(make_uint4(0u, 0u, 0u, 0u)); }

// Two floats -> one word of two bf16 (round to nearest even), first in the low
// half: one v_cvt_pk_bf16_f32.
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Pack the C values of two stacked tiles into one bf16 operand.
__device__ __forceinline__ bf16x8 pack_ctiles(const f32x4& lo, const f32x4& hi) {
  return as_bf8(make_uint4(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(hi[0], hi[1]), pack2(hi[2], hi[3])));
}

// Four floats -> 8 bytes of bf16 at p (8-byte aligned).
__device__ __forceinline__ void st4bf(void* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack2(a, b), pack2(c, d));
}

// Per-pair partial slots (forward o_b and backward dQ partials) hold R rows
// of D bf16 as 16-byte runs (run j = columns 8j .. 8j+7) in the order
// [j / 2][head][j % 2]: the two lanes that hold a row after an MFMA write
// runs 2k and 2k+1, so one 16-byte store instruction covers 32 contiguous
// bytes of each of R heads, i.e. 32 R contiguous bytes per pair.  Element
// offset of run j of head hh within a slot:
template <int R>
__device__ __forceinline__ int partial_run_offset(int hh, int j) {
  return (j >> 1) * 16 * R + 16 * hh + 8 * (j & 1);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float wave_max_xor_16_32(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float wave_sum_xor_16_32(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

}  // namespace msa
