// decode.hip -- split-KV decode: per-chunk partial triplets.
//
// The mesh decode page ("_attention_mesh_mlo.py") keeps a sequence slice of
// K/V on every rank, computes one local partial (m, l, o) against it, and then
// merges the ranks' triplets.  Here the ranks are the n_chunks chunks of each
// sequence's cache, laid side by side on one GPU: one workgroup per
// (chunk, KV head, sequence) computes the local partial of all g = h_q / h_kv
// query heads of the group at once, so every K/V byte is read from HBM once.
// The g query heads are the 32 columns of the MFMA (columns >= g are zero).
//
// The path is bandwidth-bound (8 FLOP per byte).  Each of the 4 waves streams
// its own contiguous quarter of the chunk in steps of 32 keys, with the next
// step's loads in flight while the current one computes; there is no
// workgroup barrier in the streaming loop:
//   K: each lane loads its key row's dims straight into the MFMA A operand
//      (S^T = K Q^T needs key rows, which is how K is stored);
//   V: lanes load 16-byte row chunks, transpose 4 keys x 8 dims in registers
//      and pass them through a wave-private LDS slab in the quad layout, from
//      which the A operand of O^T += V^T P^T is read.
// At the end the 4 waves' triplets merge (online-softmax rule) through LDS
// and wave 0 writes the chunk's triplet: m, l (n_chunks, B*h_q) and
// O unnormalised (n_chunks, B*h_q, d), the layout lse_merge consumes.
#include "fakv_device.h"
#include "fakv_kernels.h"

namespace fakv {

template <int D>
__global__ __launch_bounds__(256, 1)
void decode_partial_kernel(DecodeParams p, int g) {
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;
  constexpr int NCH = D / 8;                 // 16-byte chunks per key row
  constexpr int VTASK = 8 * NCH / 64;        // (quad, chunk) tasks per lane per 32-key step
  constexpr int SLAB = 32 * D * 2;           // bytes of one wave's V slab
  static_assert(VTASK * 64 == 8 * NCH, "V tasks must divide over the wave");

  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int c = blockIdx.x % p.n_chunks;
  const int kvh = (blockIdx.x / p.n_chunks) % p.h_kv;
  const int b = blockIdx.x / (p.n_chunks * p.h_kv);

  const int c0 = min(c * p.chunk_w, p.S);
  const int c1 = min(c0 + p.chunk_w, p.S);
  const int n = c1 - c0;
  const int per = ((n + 127) / 128) * 32;    // keys per wave, a multiple of 32
  const int w0 = min(c0 + wave * per, c1);
  const int w1 = min(w0 + per, c1);
  const int nsteps = (w1 - w0 + 31) / 32;

  // query heads of the group as B operands (column col = head kvh*g + col)
  const bool cvalid = col < g;
  const int head = kvh * g + col;
  bf16x8 qreg[DS];
  {
    const uint16_t* qp = p.q + ((size_t)b * p.h_q + head) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (cvalid) x = *reinterpret_cast<const u32x4*>(qp + 16 * s);
      qreg[s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const size_t kv_stride = (size_t)p.h_kv * D;
  const uint16_t* kbase = p.k + ((size_t)b * p.S * p.h_kv + kvh) * D;
  const uint16_t* vbase = p.v + ((size_t)b * p.S * p.h_kv + kvh) * D;
  char* slab = smem + wave * SLAB;

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m_run = neg_inf(), l_run = 0.f;

  struct Regs { u32x4 k[DS]; u32x4 v[VTASK][4]; };
  auto load = [&](int k0, Regs& R) {
    const int kr = k0 + col;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (kr < w1) x = *reinterpret_cast<const u32x4*>(kbase + (size_t)kr * kv_stride + 16 * s + 8 * half);
      R.k[s] = x;
    }
#pragma unroll
    for (int t = 0; t < VTASK; ++t) {
      const int id = lane + 64 * t;
      const int kq = id / NCH, ch = id % NCH;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = k0 + 4 * kq + j;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (r < w1) x = *reinterpret_cast<const u32x4*>(vbase + (size_t)r * kv_stride + 8 * ch);
        R.v[t][j] = x;
      }
    }
  };
  auto process = [&](int k0, const Regs& R) {
    // V -> wave slab (quad layout)
#pragma unroll
    for (int t = 0; t < VTASK; ++t) {
      const int id = lane + 64 * t;
      const int kq = id / NCH, ch = id % NCH;
      u32x4 o4[4];
      quad_transpose(R.v[t], o4);
      char* dst = slab + (kq * D + 8 * ch) * 8;
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) *reinterpret_cast<u32x4*>(dst + 16 * pc) = o4[pc];
    }
    // S^T = K Q^T (32 keys x 32 columns)
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int s = 0; s < DS; ++s) sacc = mfma32x32x16(__builtin_bit_cast(bf16x8, R.k[s]), qreg[s], sacc);
    if (k0 + 32 > w1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (key >= w1) sacc[r] = neg_inf();
      }
    }
    float mt = neg_inf();
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[r]);
    mt = fmaxf(mt, xor32(mt));
    const float m_new = fmaxf(m_run, mt * p.scale);
    const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
    const float alpha = fast_exp2((m_run - m_use) * kLog2e);
    const float mlog = m_use * kLog2e;
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(__builtin_fmaf(sacc[r], p.scale_log2, -mlog));
      sacc[r] = e;
      rs += e;
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pv[j] = sacc[8 * ks + j];
      const bf16x8 pb = pack_bf16x8(pv);
      const char* q0 = slab + ((4 * ks + half) * D) * 8;
      const char* q1 = slab + ((4 * ks + 2 + half) * D) * 8;
#pragma unroll
      for (int i = 0; i < DB; ++i) {
        const int e = 32 * i + col;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(q0 + e * 8);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(q1 + e * 8);
        const u32x4 a4 = {lo[0], lo[1], hi[0], hi[1]};
        oacc[i] = mfma32x32x16(__builtin_bit_cast(bf16x8, a4), pb, oacc[i]);
      }
    }
  };

  Regs A, Bv;
  if (nsteps > 0) load(w0, A);
  for (int st = 0; st < nsteps; st += 2) {
    if (st + 1 < nsteps) load(w0 + 32 * (st + 1), Bv);
    process(w0 + 32 * st, A);
    if (st + 1 < nsteps) {
      if (st + 2 < nsteps) load(w0 + 32 * (st + 2), A);
      process(w0 + 32 * (st + 1), Bv);
    }
  }

  // ---- merge the 4 waves' triplets (fixed order 0 <- 1 <- 2 <- 3) ----------
  const float l_tot = l_run + xor32(l_run);
  __syncthreads();                              // slabs are free from here on
  float* red = reinterpret_cast<float*>(smem);  // [wave][col][D + 2]
  constexpr int RS = D + 2;
  if (wave > 0) {
    float* dst = red + ((wave - 1) * 32 + col) * RS;
    if (half == 0) { dst[D] = m_run; dst[D + 1] = l_tot; }
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[32 * i + 8 * (r >> 2) + 4 * half + (r & 3)] = oacc[i][r];
  }
  __syncthreads();
  if (wave != 0 || !cvalid) return;
  float m = m_run, l = l_tot;
  for (int wv = 1; wv < 4; ++wv) {
    const float* src = red + ((wv - 1) * 32 + col) * RS;
    const float m2 = src[D], l2 = src[D + 1];
    const float mn = fmaxf(m, m2);
    const float mu = (mn == neg_inf()) ? 0.f : mn;
    const float a1 = fast_exp2((m - mu) * kLog2e), a2 = fast_exp2((m2 - mu) * kLog2e);
    l = l * a1 + l2 * a2;
    m = mn;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        oacc[i][r] = oacc[i][r] * a1 + src[32 * i + 8 * (r >> 2) + 4 * half + (r & 3)] * a2;
  }
  const size_t row = (size_t)b * p.h_q + head;
  const size_t rows = (size_t)p.B * p.h_q;
  if (half == 0) {
    p.m_parts[(size_t)c * rows + row] = m;
    p.l_parts[(size_t)c * rows + row] = l;
  }
  float* op = p.o_parts + ((size_t)c * rows + row) * D + 4 * half;
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f32x4 x = {oacc[i][4 * q4], oacc[i][4 * q4 + 1], oacc[i][4 * q4 + 2], oacc[i][4 * q4 + 3]};
      *reinterpret_cast<f32x4*>(op + 32 * i + 8 * q4) = x;
    }
}

template <int D>
static hipError_t launch_decode(const DecodeParams& p, int g, hipStream_t stream) {
  constexpr int slabs = 4 * 32 * D * 2;
  constexpr int red = 3 * 32 * (D + 2) * 4;
  constexpr int smem = slabs > red ? slabs : red;
  static std::atomic<unsigned> lds_done{0};
  auto kern = decode_partial_kernel<D>;
  hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), smem, lds_done);
  if (e != hipSuccess) return e;
  const long long grid = (long long)p.B * p.h_kv * p.n_chunks;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), smem, stream, p, g);
  return hipGetLastError();
}

hipError_t launch_decode_partial(const DecodeParams& p, int d, int g, hipStream_t stream) {
  switch (d) {
    case 64: return launch_decode<64>(p, g, stream);
    case 128: return launch_decode<128>(p, g, stream);
    case 256: return launch_decode<256>(p, g, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fakv
