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
// The path is bandwidth-bound (8 FLOP per byte).  Each wave owns one whole
// (sequence, KV head, chunk) unit -- a workgroup holds four -- and streams it
// in steps of 32 keys, two steps in flight, with no barrier anywhere:
//   K: each lane loads its key row's dims straight into the MFMA A operand of
//      S^T = K Q^T (key rows are how K is stored), double-buffered registers;
//   V: 32 x d tiles go HBM -> LDS directly (buffer_load ... lds, with the
//      non-temporal hint: every byte is read once) into two wave-private
//      stages, swizzled so that the A operand of O^T += V^T P^T is read with
//      the conflict-free transpose read ds_read_b64_tr_b16.
// Buffer resources span one unit's keys (one chunk of one sequence and KV
// head), so no load can leave the unit.  Each wave writes its unit's triplet: m, l
// (n_chunks, B*h_q) and O unnormalised (n_chunks, B*h_q, d), the layout
// lse_merge consumes.
#include <type_traits>
#include <utility>

#include "fakv_device.h"
#include "fakv_kernels.h"

namespace fakv {

template <int D>
__global__ __launch_bounds__(256, 2)
void decode_partial_kernel(DecodeParams p, int g) {
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;
  constexpr int NCH = D / 8;                 // 16-byte chunks per key row
  constexpr int STAGE = 32 * D * 2;          // bytes of one 32-key V stage
  constexpr int NV = 32 * NCH / 64;          // V loads per lane per step
  constexpr int NVA = DB < 4 ? DB : 4;
  constexpr int NKB = D <= 128 ? 2 : 1;      // K register buffers
  __shared__ __attribute__((aligned(16))) char smem[4 * 2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  // unit = (sequence, chunk, KV head), KV head fastest: the waves of a
  // workgroup stream neighbouring head slices of the same token rows
  const int unit = blockIdx.x * 4 + wave;
  if (unit >= p.B * p.h_kv * p.n_chunks) return;
  const int kvh = unit % p.h_kv;
  const int c = (unit / p.h_kv) % p.n_chunks;
  const int b = unit / (p.n_chunks * p.h_kv);

  const int w0 = min(c * p.chunk_w, p.S);
  const int w1 = min(w0 + p.chunk_w, p.S);
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

  const unsigned stride_b = (unsigned)p.h_kv * D * 2;
  // The resources span this unit's own keys [w0, w1) only: the loads issued
  // past its last step read zeros without touching memory.
  const size_t head_off = (((size_t)b * p.S + w0) * p.h_kv + kvh) * D;
  const unsigned extent = w1 > w0 ? (unsigned)(w1 - w0 - 1) * stride_b + D * 2 : 0u;
  const __amdgpu_buffer_rsrc_t rs_k = make_rsrc(p.k + head_off, extent);
  const __amdgpu_buffer_rsrc_t rs_v = make_rsrc(p.v + head_off, extent);
  char* wl = smem + wave * 2 * STAGE;       // this wave's two V stages

  // V stage slot l of load i holds row (64 i + l) / NCH, physical chunk (..) % NCH
  unsigned voff_v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int sl = 64 * i + lane;
    const int r = sl / NCH, pc = sl % NCH;
    voff_v[i] = (unsigned)r * stride_b + (unsigned)((pc ^ vmask<D>(r)) * 16);
  }
  const unsigned koff = (unsigned)col * stride_b + 16u * half;   // + 32 s bytes
  const lds_char* vaddr[NVA];
  {
    const int vg16 = (lane >> 4) & 1, vp = lane & 15;
    const int vrow = 4 * half + (vp >> 2);
    const int vmsk = vmask<D>(vrow);
#pragma unroll
    for (int i = 0; i < NVA; ++i)
      vaddr[i] = (const lds_char*)(wl) + vrow * (D * 2) + ((4 * i + 2 * vg16 + ((vp & 3) >> 1)) ^ vmsk) * 16 +
                 (vp & 1) * 8;
  }

  u32x4 kr[NKB][DS];
  auto issue_k = [&](int k0, int slot) {
#pragma unroll
    for (int s = 0; s < DS; ++s)
      kr[slot][s] = __builtin_amdgcn_raw_buffer_load_b128(rs_k, (int)((unsigned)(k0 - w0) * stride_b + koff + 32u * s), 0, 0);
  };
  auto issue_v = [&](int k0, int stage) {
#pragma unroll
    for (int i = 0; i < NV; ++i) dma16_stream(rs_v, (unsigned)(k0 - w0) * stride_b + voff_v[i], wl + stage * STAGE + 1024 * i);
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m_run = neg_inf(), l_run = 0.f;

  auto process = [&](int k0, auto stc) {
    constexpr int ST = decltype(stc)::value;
    // S^T = K Q^T (32 keys x 32 columns)
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int s = 0; s < DS; ++s)
      sacc = mfma32x32x16(__builtin_bit_cast(bf16x8, kr[NKB == 2 ? ST : 0][s]), qreg[s], sacc);
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
    mt = halves_max(mt);
    const float m_new = fmaxf(m_run, mt * p.scale);
    const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
    const float mlog = m_use * kLog2e;
    if (__builtin_amdgcn_ballot_w64(m_new != m_run) != 0) {
      const float alpha = fast_exp2((m_run - m_use) * kLog2e);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }
    m_run = m_new;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(__builtin_fmaf(sacc[r], p.scale_log2, -mlog));
      sacc[r] = e;
      l_run += e;
    }
    // O^T += V^T P^T from this step's V stage
    static_for<2>([&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      float pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pv[j] = sacc[8 * ks + j];
      const bf16x8 pb = pack_bf16x8(pv);
      static_for<DB / NVA>([&](auto gc) {
        constexpr int G = decltype(gc)::value;
        constexpr int OFF = ST * STAGE + 16 * ks * (D * 2) + G * 256;
        u32x2 lo[NVA], hi[NVA];
#pragma unroll
        for (int i = 0; i < NVA; ++i) {
          lo[i] = tr16_at<OFF>(vaddr[i]);
          hi[i] = tr16_at<OFF + 8 * (D * 2)>(vaddr[i]);
        }
        lds_wait();
#pragma unroll
        for (int i = 0; i < NVA; ++i) {
          lds_ready(lo[i]);
          lds_ready(hi[i]);
          const u32x4 a4 = {lo[i][0], lo[i][1], hi[i][0], hi[i][1]};
          oacc[G * NVA + i] = mfma32x32x16(__builtin_bit_cast(bf16x8, a4), pb, oacc[G * NVA + i]);
        }
      });
    });
  };

  // Step st uses K buffer st % NKB and V stage st % 2.  Loads of step st + 2
  // (st + 1 with one K buffer) are issued as soon as their buffer is free.
  // The loads are issued unconditionally -- past the unit's keys they hit
  // offsets beyond the resource, read as zero without a memory access, and
  // are never used -- so every step sees the same number of younger loads in
  // flight and the waits below are exact.
  issue_k(w0, 0);
  issue_v(w0, 0);
  if (NKB == 2) issue_k(w0 + 32, 1);
  issue_v(w0 + 32, 1);
  auto step = [&](int st, auto stc) {
    constexpr int ST = decltype(stc)::value;
    const int k0 = w0 + 32 * st;
    // this step's loads have landed once only the next step's are pending
    vm_wait<(NKB == 2 ? DS : 0) + NV>();
    process(k0, stc);
    if (NKB == 1) issue_k(k0 + 32, 0);
    if (NKB == 2) issue_k(k0 + 64, ST);
    issue_v(k0 + 64, ST);
  };
  for (int st = 0; st < nsteps; st += 2) {
    step(st, std::integral_constant<int, 0>{});
    if (st + 1 < nsteps) step(st + 1, std::integral_constant<int, 1>{});
  }

  // ---- this unit's triplet -------------------------------------------------
  const float l_tot = halves_sum(l_run);
  vm_wait<0>();                 // no load into LDS may still be in flight at exit
  if (!cvalid) return;
  const size_t row = (size_t)b * p.h_q + head;
  const size_t rows = (size_t)p.B * p.h_q;
  if (half == 0) {
    p.m_parts[(size_t)c * rows + row] = m_run;
    p.l_parts[(size_t)c * rows + row] = l_tot;
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
  const long long units = (long long)p.B * p.h_kv * p.n_chunks;
  const long long grid = (units + 3) / 4;
  hipLaunchKernelGGL(decode_partial_kernel<D>, dim3((unsigned)grid), dim3(256), 0, stream, p, g);
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
