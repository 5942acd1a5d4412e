// prefill_bf16.hip -- blockwise causal/non-causal prefill attention on gfx950
// bf16 MFMA with fp32 accumulation.
//
// One workgroup (4 waves) owns one query tile of QH query heads that share a
// KV head (GQA), 32 query rows per wave.  It walks the KV chunks in ring order
// ("_gqa_prefill_long.py": rank r holds chunk (r + s) mod C at step s) and,
// inside a chunk, the tiles of BK keys up to the dependent end
// min(chunk end, query tile end) ("[pallas] Support dependent Tile.end bounds
// in Pallas", "Unroll lowering": the trip count shrinks instead of masking
// whole tiles).  Per tile:
//   1. K and V tiles are staged HBM -> registers -> LDS (K swizzled, V
//      quad-transposed), double-buffered: tile t+1's loads are in flight
//      while tile t computes.
//   2. S^T = K Q^T on MFMA (Q resident in registers as the B operand).
//   3. The online-softmax fold of the prefill page's ring step, with the
//      block partial folded directly into the running (m, l, O): row max,
//      exp2 of pre-scaled scores, per-lane partial row sums, rescale of O.
//   4. O^T += V^T P^T on MFMA (P rounded to bf16 in registers).
// Only tiles that straddle the diagonal or the chunk's tail evaluate the
// element mask.  The epilogue writes O / l in bf16, or the fp32 triplet.
#include "fakv_device.h"
#include "fakv_kernels.h"

namespace fakv {

template <int D, int BK, int QH>
__global__ __launch_bounds__(256, (D <= 128) ? 2 : 1)
void prefill_bf16_kernel(PrefillParams p) {
  constexpr int WPH = 4 / QH;          // waves per query head
  constexpr int BQ = 32 * WPH;         // query rows per tile
  constexpr int KB = BK / 32;          // 32-key MFMA blocks per tile
  constexpr int DS = D / 16;           // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;           // 32-dim blocks of O^T
  constexpr int KS = BK / 16;          // k-steps of O^T += V^T P^T
  constexpr int TILE_BYTES = BK * D * 2;
  constexpr int NCH = D / 8;           // 16-byte chunks per key row
  constexpr int KCH = BK * NCH / 256;  // K chunks staged per thread
  constexpr int VT = (BK / 4) * NCH / 256;  // V quad tasks per thread
  static_assert(KCH * 256 == BK * NCH && VT * 256 == (BK / 4) * NCH, "tile/threads mismatch");

  extern __shared__ __attribute__((aligned(16))) char smem[];  // K0 V0 K1 V1

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = wave / WPH;
  const int qsub = wave % WPH;
  const int half = lane >> 5;
  const int col = lane & 31;

  // ---- work item -----------------------------------------------------------
  int seq_q0, seq_k0, Lq, Lk, q_lo, q_hi, hg;
  if (p.items != nullptr) {
    const int item = blockIdx.x / p.n_hg;
    hg = blockIdx.x - item * p.n_hg;
    if (item >= *p.n_items) return;
    const int32_t* it = p.items + 8 * (size_t)item;
    seq_q0 = seq_k0 = it[2];
    Lq = Lk = it[3];
    q_lo = it[4] - it[2];
    q_hi = it[6] - it[2];
  } else {
    const int pairs = p.n_seqs * p.n_hg;
    const int qt_rev = blockIdx.x / pairs;
    const int pair = blockIdx.x - qt_rev * pairs;
    const int qt = p.n_qtiles - 1 - qt_rev;      // longest (causal) tiles first
    const int seq = pair / p.n_hg;
    hg = pair - seq * p.n_hg;
    seq_q0 = seq * p.T_q;
    seq_k0 = seq * p.S_kv;
    Lq = p.T_q;
    Lk = p.S_kv;
    q_lo = qt * BQ;
    q_hi = min(q_lo + BQ, Lq);
  }
  const int head = hg * QH + hl;
  const int kvh = head / (p.h_q / p.h_kv);
  const int delta = p.q_pos0 - p.k_pos0;
  const int w = (p.items != nullptr) ? (Lk + p.C - 1) / p.C : Lk / p.C;

  KvWalk walk;
  walk.S = Lk; walk.C = p.C; walk.w = w;
  walk.r = (Lq > 0) ? (int)(((long long)q_lo * p.C) / Lq) : 0;
  walk.q_hi = q_hi; walk.delta = delta; walk.causal = p.causal; walk.prune = p.prune;
  walk.BK = BK;
  walk.first();

  // ---- query rows of this wave, resident as MFMA B operands ---------------
  const int qw_lo = q_lo + 32 * qsub;
  const int qw_hi = min(qw_lo + 32, q_hi);
  const bool wave_active = qw_lo < q_hi;
  const int qi = qw_lo + col;
  const bool qvalid = qi < q_hi;
  const size_t qrow = (size_t)(seq_q0 + qi) * p.h_q + head;

  bf16x8 qreg[DS];
  {
    const uint16_t* qp = p.q + qrow * D + 8 * half;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qvalid) x = *reinterpret_cast<const u32x4*>(qp + 16 * s);
      qreg[s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[b] = f32x16{};
  float m_run = neg_inf();   // natural-log units of the scaled score
  float l_run = 0.f;         // this lane's partial row sum (keys of its half)
  if (p.mode == 2 && qvalid) {
    m_run = p.m_st[qrow];
    l_run = half == 0 ? p.l_st[qrow] : 0.f;
    const float* os = p.o_st + qrow * D + 4 * half;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x = *reinterpret_cast<const f32x4*>(os + 32 * b + 8 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[b][4 * g + i] = x[i];
      }
  }

  // ---- staging of K/V tiles ------------------------------------------------
  const size_t kv_stride = (size_t)p.h_kv * D;           // elements between keys
  const uint16_t* kbase = p.k + ((size_t)seq_k0 * p.h_kv + kvh) * D;
  const uint16_t* vbase = p.v + ((size_t)seq_k0 * p.h_kv + kvh) * D;

  u32x4 kst[KCH];
  u32x4 vst[VT][4];
  auto load_tile = [&](int kt, int lim) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int id = tid + 256 * i;
      const int r = id / NCH, c = id % NCH;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (kt + r < lim) x = *reinterpret_cast<const u32x4*>(kbase + (size_t)(kt + r) * kv_stride + 8 * c);
      kst[i] = x;
    }
#pragma unroll
    for (int i = 0; i < VT; ++i) {
      const int id = tid + 256 * i;
      const int kq = id / NCH, c = id % NCH;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * kq + j;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (kt + r < lim) x = *reinterpret_cast<const u32x4*>(vbase + (size_t)(kt + r) * kv_stride + 8 * c);
        vst[i][j] = x;
      }
    }
  };
  auto store_tile = [&](int buf) {
    char* kl = smem + buf * 2 * TILE_BYTES;
    char* vl = kl + TILE_BYTES;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int id = tid + 256 * i;
      const int r = id / NCH, c = id % NCH;
      *reinterpret_cast<u32x4*>(kl + r * (D * 2) + kswz<D>(r, c) * 16) = kst[i];
    }
#pragma unroll
    for (int i = 0; i < VT; ++i) {
      const int id = tid + 256 * i;
      const int kq = id / NCH, c = id % NCH;
      u32x4 t[4];
      quad_transpose(vst[i], t);
      char* dst = vl + (kq * D + 8 * c) * 8;
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) *reinterpret_cast<u32x4*>(dst + 16 * pc) = t[pc];
    }
  };

  const float scale = p.scale;
  const float scale_log2 = p.scale_log2;

  if (walk.valid) {
    load_tile(walk.kt, walk.end);
    store_tile(0);
  }
  __syncthreads();

  int buf = 0;
  while (walk.valid) {
    const int kt = walk.kt;
    const int end = walk.end;
    KvWalk nxt = walk;
    nxt.next();
    if (nxt.valid) load_tile(nxt.kt, nxt.end);

    const bool skip = !wave_active || (p.causal && p.prune && kt > qw_hi - 1 + delta);
    if (!skip) {
      const char* kl = smem + buf * 2 * TILE_BYTES;
      const char* vl = kl + TILE_BYTES;
      // S^T = K Q^T
      f32x16 sacc[KB];
#pragma unroll
      for (int b = 0; b < KB; ++b) sacc[b] = f32x16{};
#pragma unroll
      for (int s = 0; s < DS; ++s) {
#pragma unroll
        for (int b = 0; b < KB; ++b) {
          const int r = 32 * b + col;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kl + r * (D * 2) + kswz<D>(r, 2 * s + half) * 16);
          sacc[b] = mfma32x32x16(a, qreg[s], sacc[b]);
        }
      }
      // element mask only on tiles that cross the tail or the diagonal
      const bool need_mask = (kt + BK > end) || (p.causal && (kt + BK - 1 > qw_lo + delta));
      if (need_mask) {
        const int qlim = qi + delta;
#pragma unroll
        for (int b = 0; b < KB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt + 32 * b + 8 * (r >> 2) + 4 * half + (r & 3);
            const bool ok = key < end && (!p.causal || key <= qlim);
            if (!ok) sacc[b][r] = neg_inf();
          }
      }
      // online softmax fold
      float mt = neg_inf();
#pragma unroll
      for (int b = 0; b < KB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[b][r]);
      mt = fmaxf(mt, xor32(mt));
      const float m_new = fmaxf(m_run, mt * scale);
      const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
      const float alpha = fast_exp2((m_run - m_use) * kLog2e);
      const float mlog = m_use * kLog2e;
      float rs = 0.f;
#pragma unroll
      for (int b = 0; b < KB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(__builtin_fmaf(sacc[b][r], scale_log2, -mlog));
          sacc[b][r] = e;
          rs += e;
        }
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
      // O^T += V^T P^T
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pv[j] = sacc[ks >> 1][8 * (ks & 1) + j];
        const bf16x8 pb = pack_bf16x8(pv);
        const char* q0 = vl + ((4 * ks + half) * D) * 8;
        const char* q1 = vl + ((4 * ks + 2 + half) * D) * 8;
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const int e = 32 * b + col;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(q0 + e * 8);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(q1 + e * 8);
          const u32x4 a4 = {lo[0], lo[1], hi[0], hi[1]};
          oacc[b] = mfma32x32x16(__builtin_bit_cast(bf16x8, a4), pb, oacc[b]);
        }
      }
    }

    if (nxt.valid) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    walk = nxt;
  }

  // ---- epilogue -------------------------------------------------------------
  const float l_tot = l_run + xor32(l_run);
  if (!qvalid) return;
  if (p.mode == 0) {
    const float inv = 1.f / l_tot;
    uint16_t* op = p.o + qrow * D + 4 * half;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 x = {pack_bf16x2(oacc[b][4 * g] * inv, oacc[b][4 * g + 1] * inv),
                   pack_bf16x2(oacc[b][4 * g + 2] * inv, oacc[b][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + 32 * b + 8 * g) = x;
      }
  } else {
    if (half == 0) {
      p.m_st[qrow] = m_run;
      p.l_st[qrow] = l_tot;
    }
    float* os = p.o_st + qrow * D + 4 * half;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x = {oacc[b][4 * g], oacc[b][4 * g + 1], oacc[b][4 * g + 2], oacc[b][4 * g + 3]};
        *reinterpret_cast<f32x4*>(os + 32 * b + 8 * g) = x;
      }
  }
}

template <int D, int BK, int QH>
static hipError_t launch_one(const PrefillParams& p, int grid, hipStream_t stream) {
  constexpr int smem = 4 * BK * D * 2;
  auto kern = prefill_bf16_kernel<D, BK, QH>;
  static std::atomic<unsigned> lds_done{0};
  hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), smem, lds_done);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), smem, stream, p);
  return hipGetLastError();
}

template <int D, int BK>
static hipError_t launch_qh(const PrefillParams& p, int qh, int grid, hipStream_t stream) {
  switch (qh) {
    case 1: return launch_one<D, BK, 1>(p, grid, stream);
    case 2: return launch_one<D, BK, 2>(p, grid, stream);
    case 4: return launch_one<D, BK, 4>(p, grid, stream);
  }
  return hipErrorInvalidValue;
}

int prefill_bf16_block_k(int d) { return d == 64 ? 128 : 64; }

hipError_t launch_prefill_bf16(const PrefillParams& p, int d, int qh, int grid, hipStream_t stream) {
  switch (d) {
    case 64: return launch_qh<64, 128>(p, qh, grid, stream);
    case 128: return launch_qh<128, 64>(p, qh, grid, stream);
    case 256: return launch_qh<256, 64>(p, qh, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fakv
