// fakv_device.h -- device helpers shared by the gfx950 kernels.
//
// MFMA operand conventions used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   A (32 x 16): lane l holds row l%32, k-columns 8*(l/32) .. +7   (8 bf16)
//   B (16 x 32): lane l holds column l%32, k-rows 8*(l/32) .. +7   (8 bf16)
//   C (32 x 32): lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
// The scores are formed transposed, S^T = K Q^T (keys on rows, queries on
// columns), so each lane owns one query column: the row max and row sum of
// the softmax reduce inside the lane plus one exchange with lane l^32, and the
// running (m, l) is a single scalar per lane.  P^T's C-layout registers are
// used directly as the B operand of O^T += V^T P^T: the contraction index
// (keys) is permuted identically on both operands, which leaves the sum
// unchanged, so no cross-lane shuffle of P is needed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace fakv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// 2^x on the hardware transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x2f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Value of the other half-wave's lane (l ^ 32), through LDS (any wave size).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// max / sum of x over lanes l and l ^ 32 with v_permlane32_swap (a VALU lane
// swap between the two half-waves, no LDS round trip).  Swapping x with
// itself leaves, in every lane, one register holding x of lane l mod 32 and
// the other holding x of lane l mod 32 + 32.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two fp32 -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32), packed.
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* p) {
  u32x4 u = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
             pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<unsigned>(x) << 16);
}

template <typename T>
__device__ __forceinline__ T ldg(const T* p) { return *p; }

// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Buffer resources and direct HBM -> LDS loads.

// Raw buffer over `bytes` bytes at `base` (gfx9 dword3: 32-bit untyped data).
// Loads at or past `bytes` return 0, so a resource bounds every access made
// through it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One 16-byte load per lane from a buffer resource straight into LDS; lane l
// writes lds_wave_base + 16 l.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, unsigned voff, char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_wave_base, 16,
                                           voff, 0, 0, 0);
}

// dma16 with the non-temporal cache policy (bit 1 of the buffer instruction's
// cache-policy operand): for data read once, such as a KV cache streamed by
// decode; measured +10 % on the decode V stream, while the same hint on the
// register loads of K slowed that stream down.
__device__ __forceinline__ void dma16_stream(__amdgpu_buffer_rsrc_t rs, unsigned voff, char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_wave_base, 16,
                                           voff, 0, 0, 2);
}

typedef __attribute__((address_space(3))) char lds_char;

// LDS transpose read ds_read_b64_tr_b16 at p + OFF, issued as inline asm so
// that outstanding HBM -> LDS loads into other buffers are not waited for
// (the compiler treats its builtin form as touching any LDS byte).  Call
// lds_wait() and then lds_ready() on the results before using them.
template <int OFF>
__device__ __forceinline__ u32x2 tr16_at(const lds_char* p) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(p), "i"(OFF));
  return r;
}
// 16-byte LDS read at p + OFF, inline asm for the same reason.
template <int OFF>
__device__ __forceinline__ u32x4 ds_read16_at(const lds_char* p) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(p), "i"(OFF));
  return r;
}
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Wait until at most N LDS reads are outstanding.  LDS reads complete in
// issue order, so the older ones are done -- valid only while no scalar
// memory load is outstanding (those share the counter but complete out of
// order); callers drain the counter with lds_wait() first.
template <int N>
__device__ __forceinline__ void lds_wait_n() { asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N) : "memory"); }
// Ties a value to the preceding lds_wait() so no use is scheduled above it.
__device__ __forceinline__ void lds_ready(u32x2& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void lds_ready(u32x4& x) { asm volatile("" : "+v"(x)); }

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(std::integral_constant<int, i>) for i = 0 .. N-1: each index a compile-time constant.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Wait until at most N vector-memory loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory"); }

// ---------------------------------------------------------------------------
// Chunk swizzles.  K: chunk c of row r at c ^ (r & 15) (c ^ (r & 7) for
// d = 64): the 16 lanes of each ds_read_b128 pass read 16 consecutive keys at
// one chunk and hit 16 distinct 16-byte bank groups.  V: rows r .. r+3 read by
// one half-wave in a transpose read land in distinct 64-byte bank groups.
template <int D>
__device__ __forceinline__ int vmask(int r) {
  if constexpr (D == 64) return ((r >> 1) & 1) << 2;
  else return (r & 3) << 2;
}
template <int D>
__device__ __forceinline__ int kmask(int r) {
  if constexpr (D == 64) return r & 7;
  else return r & 15;
}

// ---------------------------------------------------------------------------
// Walk over the KV tiles one query tile visits: ring chunks in the order
// (r + s) mod C, each chunk cut at its dependent end, tiles of BK keys.
// All fields are wave-uniform.
struct KvWalk {
  int S;          // keys of the sequence
  int C;          // ring chunks
  int w;          // chunk width
  int r;          // ring position of the query tile
  int q_hi;       // one past the tile's last query row (local index)
  int delta;      // query position - key position offset (causal: j <= i + delta)
  int causal;
  int prune;
  int BK;
  int lo;         // sliding window: first key the tile's first row admits (else very negative)
  int single;     // visit chunk r only (one part of a split-KV partial), not the whole ring
  // state
  int s;          // ring step of the current chunk
  int c0, c1;     // current chunk's key range
  int end;        // active end in the current chunk
  int kt;         // current tile start
  int valid;

  __device__ __forceinline__ bool open_chunk() {
    // Opens chunk (r + s) mod C; returns whether it has at least one tile.
    int c = r + s;
    if (c >= C) c -= C;
    c0 = min(c * w, S);
    c1 = min(c0 + w, S);
    if (causal && prune) end = min(c1, q_hi + delta);
    else end = c1;
    // dependent lower bound: start at the tile (on the chunk's grid) holding lo
    kt = c0;
    if (lo > c0) kt = c0 + ((lo - c0) / BK) * BK;
    return end > kt;
  }
  __device__ __forceinline__ void first() {
    s = 0;
    valid = 0;
    const int n = single ? 1 : C;
    for (; s < n; ++s)
      if (open_chunk()) { valid = 1; return; }
  }
  __device__ __forceinline__ void next() {
    kt += BK;
    if (kt < end) return;
    const int n = single ? 1 : C;
    for (++s; s < n; ++s)
      if (open_chunk()) return;
    valid = 0;
  }
};

}  // namespace fakv
