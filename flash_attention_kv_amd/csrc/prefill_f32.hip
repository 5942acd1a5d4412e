// prefill_f32.hip -- fp32 blockwise prefill attention (fp32 in, fp32 out).
//
// Same walk as the bf16 kernel (ring chunk order, dependent causal end, tail
// masks, jagged items, triplet modes), evaluated in fp32 end to end on the
// fp32 MFMA (v_mfma_f32_32x32x2f32: products and sums in fp32, no operand
// rounding).  With a contraction depth of 2 per instruction each lane holds a
// single k-value per operand.  In S^T = K Q^T k-step s pairs head dims s and
// s + D/2 (the lane's half picks which), so a lane's Q values and its slice
// of a K row are contiguous: Q arrives by 16-byte loads and K by 16-byte LDS
// reads, issued ahead of the MFMAs.  V needs no transposition: for the value
// product O^T += V^T P^T the lane's own P register is the B operand and V is
// read row-major, one 32-dim block ahead of its MFMAs (the first block while
// the softmax runs).  One workgroup = 4 waves = 128 query rows of one head.
//
// Split-KV mode (kv_parts = P > 0, dense batches): the ring's C chunks are cut
// into P equal parts (P a multiple of C, so every part lies inside one ring
// chunk) and each workgroup computes the partial triplet of one (query tile,
// part) -- the prefill page's per-chunk partial, spread over P workgroups
// instead of walked by one -- writing it at part * rows of the triplet
// arrays; lse_merge then folds the P parts of every row.  Small problems (one
// 128-row tile against a few hundred keys) otherwise leave all but one CU idle.
#include "fakv_device.h"
#include "fakv_kernels.h"

namespace fakv {

template <int D>
__global__ __launch_bounds__(256, 1)
void prefill_f32_kernel(PrefillParams p) {
  constexpr int BK = 32;               // keys per tile (one MFMA block)
  constexpr int BQ = 128;
  constexpr int DB = D / 32;
  constexpr int KST = D + 4;           // LDS row stride (floats) of K: 16-byte rows, 4-bank skew
  constexpr int VST = D + 8;           // LDS row stride (floats) of V
  constexpr int KBYTES = BK * KST * 4;
  constexpr int VBYTES = BK * VST * 4;
  constexpr int NCH = D / 4;           // 16-byte chunks per row
  constexpr int CH = BK * NCH / 256;   // chunks per thread per tensor
  static_assert(CH * 256 == BK * NCH, "tile/threads mismatch");

  extern __shared__ __attribute__((aligned(16))) char smem[];

  const float* Q = reinterpret_cast<const float*>(p.q);
  const float* K = reinterpret_cast<const float*>(p.k);
  const float* V = reinterpret_cast<const float*>(p.v);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;

  int seq_q0, seq_k0, Lq, Lk, q_lo, q_hi, head;
  int part = 0, wg = blockIdx.x;
  if (p.kv_parts > 0) {
    part = wg % p.kv_parts;
    wg /= p.kv_parts;
  }
  if (p.items != nullptr) {
    const int item = blockIdx.x / p.n_hg;
    head = blockIdx.x - item * p.n_hg;
    if (item >= *p.n_items) return;
    const int32_t* it = p.items + 8 * (size_t)item;
    seq_q0 = seq_k0 = it[2];
    Lq = Lk = it[3];
    q_lo = it[4] - it[2];
    q_hi = it[6] - it[2];
  } else {
    const int pairs = p.n_seqs * p.n_hg;
    const int qt_rev = wg / pairs;
    const int pair = wg - qt_rev * pairs;
    const int qt = p.n_qtiles - 1 - qt_rev;
    const int seq = pair / p.n_hg;
    head = pair - seq * p.n_hg;
    seq_q0 = seq * p.T_q; seq_k0 = seq * p.S_kv;
    Lq = p.T_q; Lk = p.S_kv;
    q_lo = qt * BQ;
    q_hi = min(q_lo + BQ, Lq);
  }
  const int kvh = head / (p.h_q / p.h_kv);
  const int delta = p.q_pos0 - p.k_pos0;
  const int w = (p.items != nullptr) ? (Lk + p.C - 1) / p.C : Lk / p.C;

  KvWalk walk;
  walk.S = Lk; walk.C = p.C; walk.w = w;
  walk.r = (Lq > 0) ? (int)(((long long)q_lo * p.C) / Lq) : 0;
  walk.q_hi = q_hi; walk.delta = delta; walk.causal = p.causal; walk.prune = p.prune;
  walk.BK = BK;
  walk.single = 0;
  if (p.kv_parts > 0) {          // this workgroup's part only
    walk.C = p.kv_parts;
    walk.w = Lk / p.kv_parts;
    walk.r = part;
    walk.single = 1;
  }
  // sliding window W (causal): key j is admissible for query i iff
  // i - W < j <= i; the walk starts at the tile holding the first row's first key
  const int win = p.causal ? p.window : 0;
  walk.lo = (win > 0 && p.prune) ? q_lo + delta - win + 1 : -(1 << 30);
  walk.first();

  const int qw_lo = q_lo + 32 * wave;
  const int qw_hi = min(qw_lo + 32, q_hi);
  const bool wave_active = qw_lo < q_hi;
  const int qi = qw_lo + col;
  const bool qvalid = qi < q_hi;
  const size_t qrow = (size_t)(seq_q0 + qi) * p.h_q + head;

  // Q^T as B operands: k-step s covers dims s and s + D/2; this lane holds
  // dim s + (D/2) half, i.e. D/2 contiguous floats.
  float qreg[D / 2];
  {
    f32x4 qv[D / 8];
#pragma unroll
    for (int i = 0; i < D / 8; ++i) qv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (qvalid) {
      const float* qp = Q + qrow * D + (D / 2) * half;
#pragma unroll
      for (int i = 0; i < D / 8; ++i) qv[i] = *reinterpret_cast<const f32x4*>(qp + 4 * i);
    }
#pragma unroll
    for (int i = 0; i < D / 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) qreg[4 * i + j] = qv[i][j];
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[b] = f32x16{};
  float m_run = neg_inf(), l_run = 0.f;
  if (p.mode == 2 && qvalid) {
    m_run = p.m_st[qrow];
    l_run = half == 0 ? p.l_st[qrow] : 0.f;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        oacc[b][r] = p.o_st[qrow * D + 32 * b + 8 * (r >> 2) + 4 * half + (r & 3)];
  }

  const size_t kv_stride = (size_t)p.h_kv * D;
  const float* kbase = K + ((size_t)seq_k0 * p.h_kv + kvh) * D;
  const float* vbase = V + ((size_t)seq_k0 * p.h_kv + kvh) * D;
  f32x4 kst[CH], vst[CH];
  auto load_tile = [&](int kt, int lim) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int id = tid + 256 * i;
      const int r = id / NCH, c = id % NCH;
      f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = a;
      if (kt + r < lim) {
        a = *reinterpret_cast<const f32x4*>(kbase + (size_t)(kt + r) * kv_stride + 4 * c);
        b = *reinterpret_cast<const f32x4*>(vbase + (size_t)(kt + r) * kv_stride + 4 * c);
      }
      kst[i] = a; vst[i] = b;
    }
  };
  auto store_tile = [&](int buf) {
    float* kl = reinterpret_cast<float*>(smem + buf * (KBYTES + VBYTES));
    float* vl = reinterpret_cast<float*>(smem + buf * (KBYTES + VBYTES) + KBYTES);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int id = tid + 256 * i;
      const int r = id / NCH, c = id % NCH;
      *reinterpret_cast<f32x4*>(kl + r * KST + 4 * c) = kst[i];
      *reinterpret_cast<f32x4*>(vl + r * VST + 4 * c) = vst[i];
    }
  };

  const float scale = p.scale, scale_log2 = p.scale_log2;
  if (walk.valid) { load_tile(walk.kt, walk.end); store_tile(0); }
  __syncthreads();

  int buf = 0;
  while (walk.valid) {
    const int kt = walk.kt, end = walk.end;
    KvWalk nxt = walk;
    nxt.next();
    if (nxt.valid) load_tile(nxt.kt, nxt.end);

    const bool skip = !wave_active || (p.causal && p.prune && kt > qw_hi - 1 + delta) ||
                      (win > 0 && p.prune && kt + BK - 1 < qw_lo + delta - win + 1);
    if (!skip) {
      const float* kl = reinterpret_cast<const float*>(smem + buf * (KBYTES + VBYTES));
      const float* vl = reinterpret_cast<const float*>(smem + buf * (KBYTES + VBYTES) + KBYTES);
      // S^T = K Q^T: the lane's K slice in 16-byte reads, KC of them (4
      // k-steps each) in flight before their MFMAs
      constexpr int KG = D / 8;
      constexpr int KC = KG < 16 ? KG : 16;
      const float* krow = kl + col * KST + (D / 2) * half;
      f32x16 sacc = f32x16{};
#pragma unroll
      for (int c0 = 0; c0 < KG; c0 += KC) {
        f32x4 kv[KC];
#pragma unroll
        for (int g = 0; g < KC; ++g) kv[g] = *reinterpret_cast<const f32x4*>(krow + 4 * (c0 + g));
#pragma unroll
        for (int g = 0; g < KC; ++g)
#pragma unroll
          for (int j = 0; j < 4; ++j) sacc = mfma32x32x2f32(kv[g][j], qreg[4 * (c0 + g) + j], sacc);
      }
      // V operands of dim block 0, in flight while the softmax runs
      float vv[2][16];
      auto read_v = [&](int b, float* dst) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 8 * (r >> 2) + 4 * half + (r & 3);
          dst[r] = vl[key * VST + 32 * b + col];
        }
      };
      read_v(0, vv[0]);
      const bool need_mask = (kt + BK > end) || (p.causal && (kt + BK - 1 > qw_lo + delta)) ||
                             (win > 0 && kt < qw_hi - 1 + delta - win + 1);
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt + 8 * (r >> 2) + 4 * half + (r & 3);
          if (!(key < end && (!p.causal || key <= qi + delta) && (win == 0 || key > qi + delta - win)))
            sacc[r] = neg_inf();
        }
      }
      float mt = neg_inf();
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[r]);
      mt = fmaxf(mt, xor32(mt));
      const float m_new = fmaxf(m_run, mt * scale);
      const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
      const float alpha = fast_exp2((m_run - m_use) * kLog2e);
      const float mlog = m_use * kLog2e;
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(__builtin_fmaf(sacc[r], scale_log2, -mlog));
        sacc[r] = e;
        rs += e;
      }
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        if (b + 1 < DB) read_v(b + 1, vv[(b + 1) & 1]);
        f32x16 acc = oacc[b] * alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc = mfma32x32x2f32(vv[b & 1][r], sacc[r], acc);
        oacc[b] = acc;
      }
    }
    if (nxt.valid) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    walk = nxt;
  }

  const float l_tot = l_run + xor32(l_run);
  if (!qvalid) return;
  float* m_st = p.m_st;
  float* l_st = p.l_st;
  float* o_st = p.o_st;
  if (p.kv_parts > 0) {
    const size_t rows = (size_t)p.n_seqs * p.T_q * p.h_q;
    m_st += part * rows;
    l_st += part * rows;
    o_st += part * rows * D;
  }
  if (p.mode == 0) {
    const float inv = 1.f / l_tot;
    float* op = reinterpret_cast<float*>(p.o) + qrow * D + 4 * half;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x = {oacc[b][4 * g] * inv, oacc[b][4 * g + 1] * inv, oacc[b][4 * g + 2] * inv,
                   oacc[b][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(op + 32 * b + 8 * g) = x;
      }
  } else {
    if (half == 0) { m_st[qrow] = m_run; l_st[qrow] = l_tot; }
    float* os = o_st + qrow * D + 4 * half;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x = {oacc[b][4 * g], oacc[b][4 * g + 1], oacc[b][4 * g + 2], oacc[b][4 * g + 3]};
        *reinterpret_cast<f32x4*>(os + 32 * b + 8 * g) = x;
      }
  }
}

template <int D>
static hipError_t launch_f32(const PrefillParams& p, int grid, hipStream_t stream) {
  constexpr int smem = 2 * (32 * (D + 4) * 4 + 32 * (D + 8) * 4);
  static std::atomic<unsigned> lds_done{0};
  auto kern = prefill_f32_kernel<D>;
  hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), smem, lds_done);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), smem, stream, p);
  return hipGetLastError();
}

hipError_t launch_prefill_f32(const PrefillParams& p, int d, int grid, hipStream_t stream) {
  switch (d) {
    case 64: return launch_f32<64>(p, grid, stream);
    case 128: return launch_f32<128>(p, grid, stream);
    case 256: return launch_f32<256>(p, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fakv
