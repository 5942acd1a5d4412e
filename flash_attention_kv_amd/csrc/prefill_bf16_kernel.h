// prefill_bf16_kernel.h -- blockwise causal/non-causal prefill attention on gfx950
// bf16 MFMA with fp32 accumulation.
//
// One workgroup (4 waves; 8 for a jagged batch) owns one query tile of QH
// query heads that share a KV head (GQA), 32 query rows per wave.  It walks the KV chunks in ring order
// ("_gqa_prefill_long.py": rank r holds chunk (r + s) mod C at step s) and,
// inside a chunk, the tiles of BK keys up to the dependent end
// min(chunk end, query tile end) ("[pallas] Support dependent Tile.end bounds
// in Pallas", "Unroll lowering": the trip count shrinks instead of masking
// whole tiles).  With a sliding window W the walk also starts late: at the
// tile holding max(chunk start, query tile start - W + 1) (the dependent
// lower bound the same page's "Scalar minimum" section leaves to
// sliding-window support).  Per tile:
//   1. K and V tiles go HBM -> LDS directly (buffer_load_dwordx4 ... lds: no
//      register staging), double-buffered: tile t+1 is in flight while tile t
//      computes.  Keys past the tile's valid end are masked.
//   2. S^T = K Q^T on MFMA (Q resident in registers as the B operand).  The
//      LDS operand reads are inline asm with explicit lgkmcnt waits, one
//      k-step ahead of the MFMAs, so that the prefetch of tile t+1 is not
//      waited for early and no read waits for the one before it.
//   3. The online-softmax fold of the prefill page's ring step, with the
//      block partial folded directly into the running (m, l, O): row max,
//      exp2 of pre-scaled scores, per-lane partial row sums.  l and O are
//      kept relative to a lazily moved shift (see kLazyShift), so O is
//      rescaled only when some row max of the wave outgrows it.
//   4. O^T += V^T P^T on MFMA: P^T straight from registers (rounded to bf16),
//      V^T read from the row-major V tile with the LDS transpose read
//      ds_read_b64_tr_b16 (a 16-lane group turns 4 keys x 16 dims into
//      16 dims x 4 keys).
// Only tiles that straddle the diagonal, a window edge or the chunk's tail
// evaluate the element mask.  The epilogue writes O / l in bf16, or the fp32
// triplet.
#pragma once

#include <type_traits>

#include "fakv_device.h"
#include "fakv_kernels.h"

namespace fakv {

// Lazy softmax shift: the running shift moves only when the row max exceeds
// it by more than this many powers of two.
constexpr float kLazyShift = 8.f;

// Keys per tile by head dim: every K or V tile is 1024 16-byte slots (16 KB).
template <int D> struct TileK { static constexpr int BK = 8192 / D; };

__device__ __forceinline__ void wait_dma_and_sync() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}


// Geometry of one work item: a query tile [q_lo, q_hi) of one sequence
// (local indices) and one head group, against that sequence's keys.
struct ItemGeo {
  int seq_q0, seq_k0;   // first query / key token of the sequence
  int Lq, Lk;           // queries / keys of the sequence
  int q_lo, q_hi;       // query tile
  int hg;               // head group
  int jagged;           // chunk width rounds up (jagged) or divides exactly (dense)
};

// One work item, start to finish: Q rows into registers, the KV walk, the
// epilogue.  The workgroup's LDS is free on entry and on exit.
template <int D, int QH, int NW>
__device__ __forceinline__ void prefill_item(const PrefillParams& p, char* smem, const ItemGeo& g) {
  constexpr int BK = TileK<D>::BK;
  constexpr int WPH = NW / QH;         // waves per query head
  constexpr int BQ = 32 * WPH;         // query rows per tile
  constexpr int KB = BK / 32;          // 32-key MFMA blocks per tile
  constexpr int DS = D / 16;           // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;           // 32-dim blocks of O^T
  constexpr int KS = BK / 16;          // k-steps of O^T += V^T P^T
  constexpr int TILE = BK * D * 2;     // bytes of one K or V tile (16 KB)
  constexpr int NCH = D / 8;           // 16-byte chunks per key row
  constexpr int NI = TILE / 16 / (64 * NW);  // DMA instructions per thread per tensor
  static_assert(TILE == 16384 && NI * 64 * NW * 16 == TILE, "tile geometry");


  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = wave / WPH;
  const int qsub = wave % WPH;
  const int half = lane >> 5;
  const int col = lane & 31;

  const int seq_q0 = g.seq_q0, seq_k0 = g.seq_k0, Lq = g.Lq, Lk = g.Lk;
  const int q_lo = g.q_lo, q_hi = g.q_hi;
  const int head = g.hg * QH + hl;
  const int kvh = head / (p.h_q / p.h_kv);
  const int delta = p.q_pos0 - p.k_pos0;
  const int w = g.jagged ? (Lk + p.C - 1) / p.C : Lk / p.C;

  KvWalk walk;
  walk.S = Lk; walk.C = p.C; walk.w = w;
  walk.r = (Lq > 0) ? (int)(((long long)q_lo * p.C) / Lq) : 0;
  walk.q_hi = q_hi; walk.delta = delta; walk.causal = p.causal; walk.prune = p.prune;
  walk.BK = BK;
  walk.single = 0;
  // sliding window W (causal): key j is admissible for query i iff
  // i - W < j <= i; the walk starts at the tile holding the first row's first key
  const int win = p.causal ? p.window : 0;
  walk.lo = (win > 0 && p.prune) ? q_lo + delta - win + 1 : -(1 << 30);
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
  // Running state.  m_true is the row max of the scaled scores seen so far;
  // l and O are kept relative to a shift m_sh <= m_true (all in natural-log
  // units of the scaled score).  The shift only moves when the max outgrows
  // it by more than kLazyShift (in log2 units), so exp terms stay <= 2^8 and
  // most tiles skip the O rescale; O / l does not depend on the shift.
  float m_true = neg_inf();
  float m_sh = neg_inf();
  float l_run = 0.f;         // this lane's partial row sum (keys of its half)
  if (p.mode == 2 && qvalid) {
    m_true = m_sh = p.m_st[qrow];
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

  // ---- direct HBM -> LDS tile loads ---------------------------------------
  // Buffer resources span this (sequence, KV head)'s rows only, so rows past
  // the sequence end read as zero (and are masked); no address can leave the
  // tensors.  The host guarantees the byte extent fits 31 bits.
  const unsigned stride_b = (unsigned)p.h_kv * D * 2;    // bytes between keys
  const size_t head_off = ((size_t)seq_k0 * p.h_kv + kvh) * D;
  const unsigned extent = Lk > 0 ? (unsigned)(Lk - 1) * stride_b + D * 2 : 0u;
  const __amdgpu_buffer_rsrc_t rs_k = make_rsrc(p.k + head_off, extent);
  const __amdgpu_buffer_rsrc_t rs_v = make_rsrc(p.v + head_off, extent);
  // slot s = (NW i + wave) * 64 + lane of a tile holds row s / NCH, physical chunk s % NCH
  unsigned voff_k[NI], voff_v[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int sl = (NW * i + wave) * 64 + lane;
    const int r = sl / NCH, pc = sl % NCH;
    voff_k[i] = (unsigned)r * stride_b + (unsigned)((pc ^ kmask<D>(r)) * 16);
    voff_v[i] = (unsigned)r * stride_b + (unsigned)((pc ^ vmask<D>(r)) * 16);
  }
  auto issue_tile = [&](int kt, int buf) {
    char* kl = smem + buf * 2 * TILE;
    char* vl = kl + TILE;
    const unsigned t0 = (unsigned)kt * stride_b;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int blk = NW * i + wave;
      dma16(rs_k, t0 + voff_k[i], kl + blk * 1024);
      dma16(rs_v, t0 + voff_v[i], vl + blk * 1024);
    }
  };

  // Lane-constant LDS read offsets (bytes within a tile).  The swizzles make
  // them non-linear in the k-step / dim block, so they are computed once here;
  // inside the loop every address is one of these plus an immediate.
  // The swizzle masks are < 16 chunks, so k-step s >= 8 (d = 256) is k-step
  // s - 8 plus 256 bytes, and dim block b >= 4 is block b - 4 plus 256 bytes:
  // KR / VR registers serve every step, the rest folds into immediates.
  constexpr int KR = DS < 8 ? DS : 8;
  constexpr int VR = DB < 4 ? DB : 4;
  int koff[KR];                                          // + 32 b rows
#pragma unroll
  for (int s = 0; s < KR; ++s) koff[s] = col * (D * 2) + (((2 * s + half) ^ kmask<D>(col)) * 16);
  int voff[VR];                                          // + 16 ks rows (+ 8 rows)
  {
    const int vg16 = (lane >> 4) & 1, vp = lane & 15;
    const int vrow = 4 * half + (vp >> 2);
    const int vmsk = vmask<D>(vrow);
#pragma unroll
    for (int b = 0; b < VR; ++b)
      voff[b] = vrow * (D * 2) + ((4 * b + 2 * vg16 + ((vp & 3) >> 1)) ^ vmsk) * 16 + (vp & 1) * 8;
  }

  const float scale = p.scale;
  const float scale_log2 = p.scale_log2;

  // One tile of the walk on LDS buffer BUF (a compile-time constant, so LDS
  // addresses fold into immediates): prefetch the next tile into the other
  // buffer, compute this one, then wait for the prefetch and synchronise.
  auto step = [&](auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const int kt = walk.kt;
    const int end = walk.end;
    KvWalk nxt = walk;
    nxt.next();
    if (nxt.valid) issue_tile(nxt.kt, BUF ^ 1);

    const bool skip = !wave_active || (p.causal && p.prune && kt > qw_hi - 1 + delta) ||
                      (win > 0 && p.prune && kt + BK - 1 < qw_lo + delta - win + 1);
    if (!skip) {
      // Every LDS read below is inline asm with explicit lgkmcnt waits: the
      // compiler would otherwise wait for the next tile's HBM -> LDS loads
      // (vmcnt(0)) before the first read of this tile, serialising prefetch
      // and compute.
      constexpr int KOFF = BUF * 2 * TILE;
      constexpr int VOFF = KOFF + TILE;
      const lds_char* lb = (const lds_char*)smem;
      lds_wait();                              // drain scalar loads: counts below are exact
      // S^T = K Q^T, K reads one k-step ahead of the MFMAs
      f32x16 sacc[KB];
#pragma unroll
      for (int b = 0; b < KB; ++b) sacc[b] = f32x16{};
      u32x4 ka[2][KB];
      static_for<KB>([&](auto bc) {
        constexpr int b = decltype(bc)::value;
        ka[0][b] = ds_read16_at<KOFF + b * 32 * (D * 2)>(lb + koff[0]);
      });
      static_for<DS>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        if constexpr (s + 1 < DS) {
          static_for<KB>([&](auto bc) {
            constexpr int b = decltype(bc)::value;
            ka[(s + 1) & 1][b] = ds_read16_at<KOFF + b * 32 * (D * 2) + ((s + 1) / 8) * 256>(lb + koff[(s + 1) % 8]);
          });
          lds_wait_n<KB>();
        } else {
          lds_wait_n<0>();
        }
        static_for<KB>([&](auto bc) {
          constexpr int b = decltype(bc)::value;
          lds_ready(ka[s & 1][b]);
          sacc[b] = mfma32x32x16(__builtin_bit_cast(bf16x8, ka[s & 1][b]), qreg[s], sacc[b]);
        });
      });
      // V^T reads go in groups of VG dim blocks (2 VG reads, within the
      // lgkmcnt range), one group ahead of the MFMAs; the first group is in
      // flight while the softmax runs.  VG is 2 at d = 256, whose O and Q
      // leave few registers for staging.
      constexpr int VG = DB < 4 ? DB : (D == 256 ? 2 : 4);
      constexpr int NG = DB / VG;
      u32x2 va[2][VG][2];
      auto issue_v = [&](auto ic, auto slotc) {
        constexpr int i = decltype(ic)::value;
        constexpr int ks = i / NG, g0 = (i % NG) * VG;
        constexpr int sl = decltype(slotc)::value;
        static_for<VG>([&](auto bc) {
          constexpr int b = decltype(bc)::value;
          constexpr int VI = VOFF + 16 * ks * (D * 2) + ((g0 + b) / 4) * 256;
          va[sl][b][0] = tr16_at<VI>(lb + voff[(g0 + b) % 4]);
          va[sl][b][1] = tr16_at<VI + 8 * (D * 2)>(lb + voff[(g0 + b) % 4]);
        });
      };
      issue_v(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
      // element mask only on tiles that cross the tail or the diagonal
      const bool need_mask = (kt + BK > end) || (p.causal && (kt + BK - 1 > qw_lo + delta)) ||
                             (win > 0 && kt < qw_hi - 1 + delta - win + 1);
      if (need_mask) {
        // Key kt + 4 half + j of register r of block b (j = 32 b + 8 (r / 4)
        // + r % 4, a constant) is admissible for the lane's row iff
        // lo < j < hi: the tail, causal and window bounds folded into two
        // per-lane limits, so each score costs one compare of j - (lo + 1)
        // against hi - lo - 1 (unsigned) and a select.
        const int qlim = qi + delta;
        const int k0 = kt + 4 * half;
        const int hi = p.causal ? min(end, qlim + 1) - k0 : end - k0;
        const int lo = win > 0 ? qlim - win - k0 : -1;
        const unsigned first = (unsigned)(lo + 1);
        const unsigned span = hi > lo + 1 ? (unsigned)(hi - lo - 1) : 0u;
#pragma unroll
        for (int b = 0; b < KB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const unsigned j = 32 * b + 8 * (r >> 2) + (r & 3);
            sacc[b][r] = j - first < span ? sacc[b][r] : neg_inf();
          }
      }
      float mt = neg_inf();
#pragma unroll
      for (int b = 0; b < KB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[b][r]);
      mt = halves_max(mt);
      m_true = fmaxf(m_true, mt * scale);
      if (__builtin_amdgcn_ballot_w64(m_true > m_sh + kLazyShift * kLn2) != 0) {
        const float mu = (m_true == neg_inf()) ? 0.f : m_true;
        const float alpha = fast_exp2((m_sh - mu) * kLog2e);
        m_sh = m_true;
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
      }
      const float mlog = ((m_sh == neg_inf()) ? 0.f : m_sh) * kLog2e;
#pragma unroll
      for (int b = 0; b < KB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(__builtin_fmaf(sacc[b][r], scale_log2, -mlog));
          sacc[b][r] = e;
          l_run += e;
        }
      // O^T += V^T P^T
      bf16x8 pb[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pv[j] = sacc[ks >> 1][8 * (ks & 1) + j];
        pb[ks] = pack_bf16x8(pv);
      }
      static_for<KS * NG>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int ks = i / NG, g0 = (i % NG) * VG;
        if constexpr (i + 1 < KS * NG) {
          issue_v(std::integral_constant<int, i + 1>{}, std::integral_constant<int, (i + 1) & 1>{});
          lds_wait_n<2 * VG>();
        } else {
          lds_wait_n<0>();
        }
        static_for<VG>([&](auto bc) {
          constexpr int b = decltype(bc)::value;
          lds_ready(va[i & 1][b][0]);
          lds_ready(va[i & 1][b][1]);
          const u32x4 a4 = {va[i & 1][b][0][0], va[i & 1][b][0][1], va[i & 1][b][1][0], va[i & 1][b][1][1]};
          oacc[g0 + b] = mfma32x32x16(__builtin_bit_cast(bf16x8, a4), pb[ks], oacc[g0 + b]);
        });
      });
    }
    wait_dma_and_sync();
    walk = nxt;
  };

  if (walk.valid) issue_tile(walk.kt, 0);
  wait_dma_and_sync();
  while (walk.valid) {
    step(std::integral_constant<int, 0>{});
    if (!walk.valid) break;
    step(std::integral_constant<int, 1>{});
  }

  // ---- epilogue -------------------------------------------------------------
  float l_tot = halves_sum(l_run);
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
    // exported triplets are relative to the true row max
    const float f = (m_true == neg_inf()) ? 1.f : fast_exp2((m_sh - m_true) * kLog2e);
    l_tot *= f;
    if (half == 0) {
      p.m_st[qrow] = m_true;
      p.l_st[qrow] = l_tot;
    }
    float* os = p.o_st + qrow * D + 4 * half;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x = {oacc[b][4 * g] * f, oacc[b][4 * g + 1] * f, oacc[b][4 * g + 2] * f, oacc[b][4 * g + 3] * f};
        *reinterpret_cast<f32x4*>(os + 32 * b + 8 * g) = x;
      }
  }
}

// Dense batches run 4 waves per workgroup (two workgroups per CU); jagged
// batches run 8 (one per CU): two query tiles' worth of rows share every K/V
// tile brought into LDS -- the "grouping 2" of the Helion page's flattened
// worklists -- which halves the tile loads per FLOP on the many short tiles
// of a jagged batch (measured +3 % there, -3 % on the dense d = 256 batch).
constexpr int kWavesDense = 4;
constexpr int kWavesJagged = 8;

// JAG instances run jagged batches only (persistent, p.sched set), the others
// dense batches only; each instance holds just its own path, which keeps the
// other path's registers out of its allocation.
template <int D, int QH, int NW, bool JAG>
__global__ __launch_bounds__(64 * NW, 8 / NW)
void prefill_bf16_kernel(PrefillParams p) {
  constexpr int BQ = 32 * (NW / QH);
  __shared__ __attribute__((aligned(16))) char smem[4 * 16384];  // K0 V0 K1 V1

  if constexpr (JAG) {
    // Jagged batch, persistent and statically scheduled.  Queue x holds the
    // entries (item * n_hg + head group) meant for XCD x -- workgroup L runs
    // on XCD L % 8 -- as whole (sequence, head group) units, longest first,
    // so the query tiles that share one sequence's K/V run on one XCD and
    // hit its L2.  The grid is a multiple of 8; the G / 8 workgroups of XCD x
    // deal the entries of queue x among themselves in zigzag rounds.  No
    // atomics: every workgroup knows its entries.  The next item's record
    // and the entry after it come in with one vector load issued before the
    // current item runs -- lanes 0..3 fetch record words 2, 3, 4 and 6, lane
    // 4 the queue entry, so the value is not uniform and stays in a vector
    // register until it is read after the item: the chain entry -> record
    // never stalls an item's start.
    const int x = blockIdx.x & 7;
    const int nj = gridDim.x >> 3;
    const int len = p.qinfo[x];
    const int32_t* q = p.sched + (size_t)x * p.sched_stride;
    const int lane = threadIdx.x & 63;
    // Round r covers slots [r nj, (r + 1) nj); workgroup j takes slot j of
    // even rounds and slot nj - 1 - j of odd ones, so a workgroup that drew a
    // long tile of a unit draws a short one next.
    const int j = blockIdx.x >> 3;
    auto slot_of = [&](int r) { return r * nj + ((r & 1) ? nj - 1 - j : j); };
    // record of the item of entry e (item 0 when e < 0, read and ignored) and
    // the entry at slot (entry 0 when slot >= len, read and ignored)
    auto fetch = [&](int e, int slot) {
      const int32_t* it = p.items + 8 * (size_t)(e >= 0 ? e / p.n_hg : 0);
      const int li = lane & 7;
      const int32_t* a = li == 0 ? it + 2 : li == 1 ? it + 3 : li == 2 ? it + 4 : li == 3 ? it + 6
                                                                        : q + (slot < len ? slot : 0);
      return *a;
    };
    struct Rec { int s0, L, lo, hi; };
    auto rec_of = [&](int v) {
      return Rec{__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 1),
                 __builtin_amdgcn_readlane(v, 2), __builtin_amdgcn_readlane(v, 3)};
    };
    auto entry_of = [&](int v, int slot) { return slot < len ? __builtin_amdgcn_readlane(v, 4) : -1; };
    if (slot_of(0) >= len) return;
    int e0 = q[slot_of(0)];
    const int v0 = fetch(e0, slot_of(1));
    Rec rc = rec_of(v0);
    int e1 = entry_of(v0, slot_of(1));
    for (int r = 0;; ++r) {
      const int vn = fetch(e1, slot_of(r + 2));   // record of item r + 1, entry of item r + 2
      ItemGeo g;
      g.seq_q0 = g.seq_k0 = rc.s0;
      g.Lq = g.Lk = rc.L;
      g.q_lo = rc.lo - rc.s0;
      g.q_hi = rc.hi - rc.s0;
      g.hg = e0 % p.n_hg;
      g.jagged = 1;
      prefill_item<D, QH, NW>(p, smem, g);
      if (e1 < 0) break;
      rc = rec_of(vn);
      e0 = e1;
      e1 = entry_of(vn, slot_of(r + 2));
    }
  } else {
    // Dense batch, one query tile per workgroup.  XCD-aware order: workgroups
    // are dispatched round-robin over the 8 XCDs (workgroup L runs on XCD
    // L % 8).  Group g of (sequence, head-group) pairs p = 8g .. 8g+7 places
    // pair 8g + x on XCD x, so all query tiles of one pair -- which read the
    // same K/V -- run on one XCD and share its L2; within a pair the longest
    // causal tiles go first.
    const int pairs = p.n_seqs * p.n_hg;
    const int main_pairs = pairs & ~7;
    const int L = blockIdx.x;
    int pair, qr;
    if (L < main_pairs * p.n_qtiles) {
      const int slot = L >> 3;
      const int pl = slot / p.n_qtiles;
      qr = slot - pl * p.n_qtiles;
      pair = pl * 8 + (L & 7);
    } else {
      const int R = L - main_pairs * p.n_qtiles;
      const int rp = pairs - main_pairs;
      qr = R / rp;
      pair = main_pairs + (R - qr * rp);
    }
    const int qt = p.n_qtiles - 1 - qr;
    const int seq = pair / p.n_hg;
    ItemGeo g;
    g.hg = pair - seq * p.n_hg;
    g.seq_q0 = seq * p.T_q;
    g.seq_k0 = seq * p.S_kv;
    g.Lq = p.T_q;
    g.Lk = p.S_kv;
    g.q_lo = qt * BQ;
    g.q_hi = min(g.q_lo + BQ, g.Lq);
    g.jagged = 0;
    prefill_item<D, QH, NW>(p, smem, g);
  }
}

template <int D, int QH, bool JAG>
inline hipError_t launch_one(const PrefillParams& p, int grid, hipStream_t stream) {
  constexpr int NW = JAG ? kWavesJagged : kWavesDense;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, QH, NW, JAG>), dim3(grid), dim3(64 * NW), 0, stream, p);
  return hipGetLastError();
}

// JAG: the persistent instances of jagged batches (p.sched set), else the dense ones
template <int D, bool JAG>
inline hipError_t launch_qh(const PrefillParams& p, int qh, int grid, hipStream_t stream) {
  switch (qh) {
    case 1: return launch_one<D, 1, JAG>(p, grid, stream);
    case 2: return launch_one<D, 2, JAG>(p, grid, stream);
    case 4: return launch_one<D, 4, JAG>(p, grid, stream);
  }
  return hipErrorInvalidValue;
}

template <int D, int QH>
inline int resident_per_cu() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_bf16_kernel<D, QH, kWavesJagged, true>,
                                                   64 * kWavesJagged, 0) != hipSuccess)
    n = 1;
  return n > 0 ? n : 1;
}

template <int D>
inline int resident_qh(int qh) {
  switch (qh) {
    case 1: return resident_per_cu<D, 1>();
    case 2: return resident_per_cu<D, 2>();
    default: return resident_per_cu<D, 4>();
  }
}

}  // namespace fakv
