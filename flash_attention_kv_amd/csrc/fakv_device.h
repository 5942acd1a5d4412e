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
// K tile in LDS: row = one key (D bf16 = D/8 chunks of 16 B).  Chunk c of row
// r lives at chunk position c ^ f(r), so the 32 lanes of an A-operand read
// (32 consecutive keys, one chunk) hit distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int kswz(int r, int c) {
  if constexpr (D == 64) return c ^ (r & 7);
  else return c ^ (r & 15);
}

// V tile in LDS, "quad-transposed": for every group of 4 consecutive keys
// (a quad) and every dimension e, the 4 bf16 values V[4q .. 4q+3][e] are
// stored together (8 bytes) at byte offset (q * D + e) * 8.  An A-operand read
// of V^T then takes two 8-byte loads per lane (keys 4h..4h+3 and 8+4h..8+4h+3
// of a 16-key step), and 32 lanes read 32 consecutive dimensions.
//
// Transpose 4 keys x 8 dims (4 x 16-byte chunks, one per key) into the quad
// layout: out[p] holds dims 2p and 2p+1, each as (keys 0-1, keys 2-3).
__device__ __forceinline__ void quad_transpose(const u32x4 in[4], u32x4 out[4]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    unsigned a = in[0][p], b = in[1][p], c = in[2][p], d = in[3][p];
    out[p][0] = (a & 0xffffu) | (b << 16);          // dim 2p,   keys 0,1
    out[p][1] = (c & 0xffffu) | (d << 16);          // dim 2p,   keys 2,3
    out[p][2] = (a >> 16) | (b & 0xffff0000u);      // dim 2p+1, keys 0,1
    out[p][3] = (c >> 16) | (d & 0xffff0000u);      // dim 2p+1, keys 2,3
  }
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
    kt = c0;
    return end > c0;
  }
  __device__ __forceinline__ void first() {
    s = 0;
    valid = 0;
    for (; s < C; ++s)
      if (open_chunk()) { valid = 1; return; }
  }
  __device__ __forceinline__ void next() {
    kt += BK;
    if (kt < end) return;
    for (++s; s < C; ++s)
      if (open_chunk()) return;
    valid = 0;
  }
};

}  // namespace fakv
