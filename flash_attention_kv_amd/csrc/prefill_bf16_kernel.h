// prefill_bf16_kernel.h -- blockwise causal/non-causal prefill attention on gfx950
// bf16 MFMA with fp32 accumulation.
//
// One workgroup of 4 waves owns one query tile of QH query heads that share a
// KV head (GQA), 32 query rows per wave; jagged batches run persistent 8-wave
// workgroups that take such work items one after another (the JAG path of
// prefill_bf16_kernel).  A work item walks the KV chunks in ring order
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

// Keys per tile: 16 KB per K or V tile (8192 / d keys), except for the dense
// d = 128 instances of 8 waves, which take 128-key (32 KB) tiles -- half the
// per-tile barriers, row-max reductions and shift checks per FLOP.
template <int D, int NW, bool JAG> struct TileK {
  static constexpr int BK = (!JAG && D == 128 && NW == 8) ? 128 : 8192 / D;
};

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

struct NoStepHook {
  __device__ void operator()(int, bool) const {}
};
struct NoNextItem {
  __device__ bool operator()(ItemGeo&) const { return false; }
};

// One work item, start to finish: Q rows into registers, the KV walk, the
// epilogue.  The K/V stages in LDS are free on entry and on exit (qstage
// below carries Q rows from one item to the next).
// on_step(i, last) runs in every wave during tile i of the walk (last: the
// item's last tile), before that tile's final barrier; an item without tiles
// still calls it once, as (0, true).
// EARLY (persistent jagged workgroups, d <= 128): every wave brings its Q
// rows through its own d/16 KB of qstage (whole-row loads, read back into
// registers before the item's first barrier).  A wave that no later tile of
// the walk concerns -- one ring chunk, causal, pruned, so key tiles come in
// increasing order and a tile past the wave's last row ends its share --
// writes its output at once and, from the third tile on (the next item's
// record is published by the end of the second), copies the Q rows it will
// have in next_item()'s geometry HBM -> LDS into its own d/16 KB of qstage,
// setting q_ready: the next item then reads them from LDS.  Those waves sit
// out the item's last diagonal tiles anyway, so the next item waits on fewer
// loads and the output stores overlap the remaining tiles.
// JAGW: the item runs in a persistent workgroup, whose next item follows at
// once (no LDS of the K/V stages is free after the walk).
template <int D, int QH, int NW, int BK, bool EARLY = false, bool JAGW = false, class StepHook = NoStepHook,
          class NextItem = NoNextItem>
__device__ __forceinline__ void prefill_item(const PrefillParams& p, char* smem, const ItemGeo& g, bool& q_ready,
                                             StepHook on_step = StepHook{}, NextItem next_item = NextItem{},
                                             char* qstage = nullptr) {
  constexpr int WPH = NW / QH;         // waves per query head
  constexpr int BQ = 32 * WPH;         // query rows per tile
  constexpr int KB = BK / 32;          // 32-key MFMA blocks per tile
  constexpr int DS = D / 16;           // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;           // 32-dim blocks of O^T
  constexpr int KS = BK / 16;          // k-steps of O^T += V^T P^T
  constexpr int TILE = BK * D * 2;     // bytes of one K or V tile (16 or 32 KB)
  constexpr int NCH = D / 8;           // 16-byte chunks per key row
  constexpr int NI = TILE / 16 / (64 * NW);  // DMA instructions per thread per tensor
  static_assert((TILE == 16384 || TILE == 32768) && NI * 64 * NW * 16 == TILE, "tile geometry");
  static_assert(!EARLY || D <= 128, "early hand-over needs the LDS of d <= 128");

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

  // Dense workgroups bring their Q rows HBM -> LDS into a wave-private slice
  // of stage 1 (free until the first step loads tile 1 there) and read them
  // into registers before the first barrier: whole-row loads instead of 32
  // bytes of each of 32 rows per instruction (+0.8 % on the GQA ring shape,
  // +1.3 % with a sliding window).  Persistent workgroups, and d = 256 whose
  // stage is too small, load them straight into registers.
  constexpr bool QSTAGE = !JAGW && NW * 32 <= 2 * BK;
  char* const qbuf = smem + 2 * TILE + wave * (32 * D * 2);

  // this wave's Q rows of item gg, into registers
  bf16x8 qreg[DS];
  auto load_q = [&](const ItemGeo& gg) {
    const int qi_g = gg.q_lo + 32 * qsub + col;
    const bool valid_g = qi_g < gg.q_hi;
    const size_t row_g = (size_t)(gg.seq_q0 + qi_g) * p.h_q + gg.hg * QH + hl;
    const uint16_t* qp = p.q + row_g * D + 8 * half;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (valid_g) x = *reinterpret_cast<const u32x4*>(qp + 16 * s);
      qreg[s] = __builtin_bit_cast(bf16x8, x);
    }
  };
  // ... or HBM -> LDS, into this wave's DS KB of qstage by whole-row loads
  // (lane l of load i brings 16 bytes of row r = RPI i + l / LPR: full
  // 128-byte lines, not 32 bytes of each of 32 rows), chunk c of row r
  // landing at r * 2d + 16 (c ^ kmask(r)); rows past the tile read 0.
  // read_stage() then takes the register layout out of it without bank
  // conflicts.  Measured +1.6 % on the jagged mix against the register loads.
  auto stage_q = [&](const ItemGeo& gg) {
    const int r0 = gg.q_lo + 32 * qsub;
    const int nr = min(32, gg.q_hi - r0);
    const unsigned rstride = (unsigned)p.h_q * D * 2;
    const unsigned ext = nr > 0 ? (unsigned)(nr - 1) * rstride + D * 2 : 0u;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(p.q + ((size_t)(gg.seq_q0 + r0) * p.h_q + gg.hg * QH + hl) * D, ext);
    constexpr int RPI = 1024 / (2 * D);
    constexpr int LPR = 64 / RPI;
#pragma unroll
    for (int i = 0; i < DS; ++i) {
      const int r = RPI * i + lane / LPR, c = (lane % LPR) ^ kmask<D>(r);
      dma16(rs, (unsigned)r * rstride + 16u * c, qstage + wave * (DS * 1024) + 1024 * i);
    }
  };
  auto read_stage = [&]() {
    const char* src = qstage + wave * (DS * 1024) + col * (2 * D);
#pragma unroll
    for (int s = 0; s < DS; ++s)
      qreg[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src + 16 * ((2 * s + half) ^ kmask<D>(col))));
  };
  bool q_lds = false;                  // rows of this item still on their way to qstage
  if constexpr (EARLY) {
    if (q_ready) {
      read_stage();
    } else {
      stage_q(g);
      q_lds = true;
    }
  } else if constexpr (!QSTAGE) {
    load_q(g);
  }
  q_ready = false;
  if constexpr (QSTAGE) {
    // lane l of DMA i brings 16 bytes of row r = RPI i + l / LPR: whole rows
    // (full 128-byte lines) per instruction, chunk c of row r landing at
    // r * 2d + 16 (c ^ kmask(r)) of the wave's slice; rows past the tile
    // fall outside the resource and read as zero
    constexpr int RPI = 1024 / (2 * D);
    constexpr int LPR = 64 / RPI;
    const int nr = min(32, q_hi - qw_lo);
    const unsigned rstride = (unsigned)p.h_q * D * 2;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + ((size_t)(seq_q0 + qw_lo) * p.h_q + head) * D,
                                                nr > 0 ? (unsigned)(nr - 1) * rstride + D * 2 : 0u);
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = RPI * i + lane / LPR, c = (lane % LPR) ^ kmask<D>(r);
      dma16(rq, (unsigned)r * rstride + 16u * c, qbuf + 1024 * i);
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

  // ---- epilogue: O / l in bf16, or the fp32 triplet ------------------------
  // Dense workgroups pass their bf16 rows through a wave-private 32 x d slice
  // of the K/V stages (free once the walk is over), so that each store
  // instruction writes whole rows -- full 128-byte lines -- instead of 16
  // bytes of each of 32 rows (measured +1.4 % on the GQA ring shape, +2.5 %
  // on the dense d = 256 batch).  Persistent jagged workgroups store straight
  // from registers: the next item's loads reuse the stages at once, and on
  // their wave-private Q hand-over region the same staging measured -0.8 %.
  constexpr bool OSTAGE = !JAGW && NW * 32 <= 4 * BK;
  char* const obuf = smem + wave * (32 * D * 2);
  auto epilogue = [&]() {
    float l_tot = halves_sum(l_run);
    if constexpr (OSTAGE) {
      if (p.mode == 0) {
        const float inv = 1.f / l_tot;           // lanes past the tile: never stored
        // lane (col, half) holds dims 32 b + 8 g + 4 half .. + 3 of row col;
        // chunk c (dims 8 c .. 8 c + 7) of row r sits at r * 2d + 16 (c ^ kmask(r)).
        // The lane index is made opaque so that the lane-dependent addresses
        // are formed here, not kept in registers across the whole tile loop.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int ocol = ln & 31;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            u32x2 x = {pack_bf16x2(oacc[b][4 * g] * inv, oacc[b][4 * g + 1] * inv),
                       pack_bf16x2(oacc[b][4 * g + 2] * inv, oacc[b][4 * g + 3] * inv)};
            *reinterpret_cast<u32x2*>(obuf + ocol * (2 * D) + 16 * ((4 * b + g) ^ kmask<D>(ocol)) + 8 * half) = x;
          }
        lds_wait();
        constexpr int RPI = 1024 / (2 * D);      // rows per 1 KB store instruction
        constexpr int LPR = 64 / RPI;            // lanes per row (its 16-byte chunks)
        const int nr = min(32, q_hi - qw_lo);
        uint16_t* orow = p.o + ((size_t)(seq_q0 + qw_lo) * p.h_q + head) * D;
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
          const int r = RPI * i + ln / LPR, c = ln % LPR;
          const u32x4 x = *reinterpret_cast<const u32x4*>(obuf + r * (2 * D) + 16 * (c ^ kmask<D>(r)));
          if (r < nr) *reinterpret_cast<u32x4*>(orow + (size_t)r * p.h_q * D + 8 * c) = x;
        }
        return;
      }
    }
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
  };
  bool epi_done = false;
  const bool early_ok = EARLY && p.C == 1 && p.causal && p.prune;
  int sidx = 0;

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
    if constexpr (EARLY) {
      if (early_ok && (!wave_active || kt > qw_hi - 1 + delta)) {   // no tile from here on is this wave's
        if (!epi_done) {
          epilogue();
          epi_done = true;
        }
        ItemGeo ng;
        if (!q_ready && sidx >= 2 && next_item(ng)) {
          stage_q(ng);
          q_ready = true;
        }
      }
    }

    const bool skip = !wave_active || (p.causal && p.prune && kt > qw_hi - 1 + delta) ||
                      (win > 0 && p.prune && kt + BK - 1 < qw_lo + delta - win + 1);
    if (!skip) {
      // Every LDS read below is inline asm with explicit lgkmcnt waits: the
      // compiler would otherwise wait for the next tile's HBM -> LDS loads
      // (vmcnt(0)) before the first read of this tile, serialising prefetch
      // and compute.
      // ds_read offsets are 16-bit immediates: with 32 KB tiles buffer 1
      // starts past them, so its reads take that base from the address register
      constexpr int BASE = 4 * TILE > 65536 ? BUF * 2 * TILE : 0;
      constexpr int KOFF = BUF * 2 * TILE - BASE;
      constexpr int VOFF = KOFF + TILE;
      const lds_char* lb = (const lds_char*)smem + BASE;
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
    on_step(sidx, !nxt.valid);
    ++sidx;
    wait_dma_and_sync();
    walk = nxt;
  };

  if (walk.valid) issue_tile(walk.kt, 0);
  else on_step(0, true);                     // no tile: the hook still runs once
  if constexpr (EARLY) {
    // the wave's own staging region: read before the barrier like the dense one
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (q_lds) {
      read_stage();
      lds_wait();
    }
    __syncthreads();
  } else if constexpr (QSTAGE) {
    // read before the barrier: past it, other waves load tile 1 into stage 1
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int s = 0; s < DS; ++s)
      qreg[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                               qbuf + col * (2 * D) + 16 * ((2 * s + half) ^ kmask<D>(col))));
    lds_wait();
    __syncthreads();
  } else {
    wait_dma_and_sync();
  }
  while (walk.valid) {
    step(std::integral_constant<int, 0>{});
    if (!walk.valid) break;
    step(std::integral_constant<int, 1>{});
  }

  if (!epi_done) epilogue();
}

// Dense batches run 4 waves per workgroup (two workgroups per CU), except at
// d = 128 without a sliding window: 8 waves (one per CU) on 128-key tiles,
// whose two 64 KB K/V stages leave no room for a second workgroup (measured
// -4 % time on the 8192-token GQA ring shape, but +5 % with a 2048-key window,
// whose edge tiles the longer tiles mask more of); jagged batches run 8 (one
// per CU):
// two query tiles' worth of rows share every K/V tile brought into LDS --
// the "grouping 2" of the Helion page's flattened worklists -- which halves
// the tile loads per FLOP on the many short tiles of a jagged batch
// (measured +3 % there, -3 % on the dense d = 256 batch).
constexpr int kWavesDense = 4;
constexpr int kWavesJagged = 8;
inline int dense_waves(int d, bool window) { return d == 128 && !window ? 8 : kWavesDense; }

// JAG instances run jagged batches only (persistent, p.sched set), the others
// dense batches only; each instance holds just its own path, which keeps the
// other path's registers out of its allocation.
template <int D, int QH, int NW, bool JAG>
__global__ __launch_bounds__(64 * NW, 8 / NW)
void prefill_bf16_kernel(PrefillParams p) {
  constexpr int BQ = 32 * (NW / QH);
  constexpr int BK = TileK<D, NW, JAG>::BK;
  __shared__ __attribute__((aligned(16))) char smem[4 * BK * D * 2];  // K0 V0 K1 V1

  if constexpr (JAG) {
    // Jagged batch, persistent, drained dynamically.  Queue x holds the
    // entries (item * n_hg + head group) meant for XCD x -- workgroup L runs
    // on XCD L % 8 -- as whole (sequence, head group) units, longest first,
    // so the query tiles that share one sequence's K/V run on one XCD and
    // hit its L2 (the worklist of the Helion page's "Flattened worklists",
    // dealt per XCD).  The workgroups of XCD x take queue x's entries in order
    // through an atomic counter, so each one takes the longest entry left
    // whenever it finishes an item, and a workgroup whose queue runs dry
    // takes entries from the next queues: the XCDs finish together instead of
    // each workgroup running a fixed share.
    //
    // Only wave 0 touches the queues, three items ahead, so no request is
    // waited for where it was issued: when item r starts it reads the record
    // of item r + 1 (its entry came in during item r - 1), reads the entry of
    // item r + 2 (its counter came in during item r - 1) and pops the counter
    // of item r + 3.  During item r's second tile (its only one, if so) --
    // before that tile's final barrier -- it publishes item r + 1's record in
    // LDS: waves done with item r early load their next Q rows from it, and
    // every wave reads it once item r is done.
    __shared__ int mbox[2][8];                      // s0, L, lo, hi, head group, valid, item number
    const int lane = threadIdx.x & 63;
    const bool w0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0;
    int32_t* cnt = p.qinfo + 16;                    // pop counter of queue q at cnt[4 q], zeroed by the scheduler
    auto qlen = [&](int qq) { return p.qinfo[qq]; };
    auto qent = [&](int qq, int slot) { return p.sched + (size_t)qq * p.sched_stride + slot; };
    int pq = blockIdx.x & 7;                        // queue being drained
    unsigned dry = 0;                               // queues found empty (bit mask)
    // Lane 0 pops queue pq; the old count lands in a vector register, read later.
    auto pop = [&]() {
      int v = 0;
      if (lane == 0) v = atomicAdd(cnt + 4 * pq, 1);
      return v;
    };
    // A popped slot of queue pq, or (when pq has run dry) a slot popped from
    // the next queue not yet found empty, at once; -1 once every queue is empty.
    auto resolve = [&](int s) {
      while (s >= qlen(pq)) {
        dry |= 1u << pq;
        if (dry == 0xFFu) return -1;
        int k = 1;
        while (dry & (1u << ((pq + k) & 7))) ++k;
        pq = (pq + k) & 7;
        s = __builtin_amdgcn_readfirstlane(pop());
      }
      return s;
    };
    // The entry at slot s of queue pq in lane 0; the other lanes read slot 0,
    // so the address is not uniform and the value stays in a vector register.
    auto entry_load = [&](int s) { return *qent(pq, lane == 0 ? s : 0); };
    // Lanes 0..3: words 2, 3, 4, 6 of the record of entry e's item.
    auto rec_load = [&](int e) {
      const int32_t* it = p.items + 8 * (size_t)(e / p.n_hg);
      const int li = lane & 3;
      return it[li == 0 ? 2 : li == 1 ? 3 : li == 2 ? 4 : 6];
    };
    auto publish_rec = [&](int* mo, bool ok, int rv, int e, int item) {
      if (lane == 0) {
        mo[0] = ok ? __builtin_amdgcn_readlane(rv, 0) : 0;
        mo[1] = ok ? __builtin_amdgcn_readlane(rv, 1) : 0;
        mo[2] = ok ? __builtin_amdgcn_readlane(rv, 2) : 0;
        mo[3] = ok ? __builtin_amdgcn_readlane(rv, 3) : 0;
        mo[4] = ok ? e % p.n_hg : 0;
        mo[5] = ok;
        mo[6] = item;
      }
    };
    auto read_geo = [&](const int* mb, ItemGeo& g) {
      g.seq_q0 = g.seq_k0 = mb[0];
      g.Lq = g.Lk = mb[1];
      g.q_lo = mb[2] - mb[0];
      g.q_hi = mb[3] - mb[0];
      g.hg = mb[4];
      g.jagged = 1;
    };
    // wave 0's pipeline: ev = entry of the next item but one (lane 0), pv = a
    // pending pop for the item after that
    int ev = 0, pv = 0;
    bool ev_ok = false, pv_ok = false;
    if (w0) {                                       // item 0 at once, item 1's entry and item 2's pop in flight
      const int s0 = resolve(__builtin_amdgcn_readfirstlane(pop()));
      const int e0 = s0 >= 0 ? __builtin_amdgcn_readlane(entry_load(s0), 0) : 0;
      publish_rec(mbox[0], s0 >= 0, s0 >= 0 ? rec_load(e0) : 0, e0, 0);
      if (lane == 0) mbox[1][6] = -1;
      if (s0 >= 0) {
        const int s1 = resolve(__builtin_amdgcn_readfirstlane(pop()));
        if (s1 >= 0) {
          ev = entry_load(s1);
          ev_ok = true;
          pv = pop();
          pv_ok = true;
        }
      }
    }
    // each wave's Q rows of its next item, when it finished the current one early
    constexpr int QST = D <= 128 ? NW * (D / 16) * 1024 : 16;
    __shared__ __attribute__((aligned(16))) char qst[QST];
    __syncthreads();
    bool q_ready = false;                           // this wave's rows of item r are in qst
    for (int r = 0;; ++r) {
      const int* mb = mbox[r & 1];
      if (!mb[5]) break;
      ItemGeo g;
      read_geo(mb, g);
      int rv = 0, e1 = 0;
      bool ok1 = false;
      if (w0) {
        ok1 = ev_ok;                                // item r + 1: its record
        if (ok1) {
          e1 = __builtin_amdgcn_readlane(ev, 0);
          rv = rec_load(e1);
        }
        ev_ok = false;                              // item r + 2: its entry, then item r + 3's pop
        if (pv_ok) {
          const int s2 = resolve(__builtin_amdgcn_readfirstlane(pv));
          if (s2 >= 0) {
            ev = entry_load(s2);
            ev_ok = true;
            pv = pop();
          }
        }
        pv_ok = ev_ok;
      }
      int* mo = mbox[(r + 1) & 1];
      bool published = false;
      prefill_item<D, QH, NW, BK, (D <= 128), true>(
          p, smem, g, q_ready,
          [&](int i, bool last) {
            if (w0 && !published && (i >= 1 || last)) {
              publish_rec(mo, ok1, rv, e1, r + 1);
              published = true;
            }
          },
          [&](ItemGeo& ng) {
            if (mo[6] != r + 1 || !mo[5]) return false;
            read_geo(mo, ng);
            return true;
          },
          qst);
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
    bool q_ready = false;
    prefill_item<D, QH, NW, BK>(p, smem, g, q_ready);
  }
}

template <int D, int QH, int NW, bool JAG>
inline hipError_t launch_one(const PrefillParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_bf16_kernel<D, QH, NW, JAG>), dim3(grid), dim3(64 * NW), 0, stream, p);
  return hipGetLastError();
}

template <int D, int QH, bool JAG>
inline hipError_t launch_nw(const PrefillParams& p, int grid, hipStream_t stream) {
  if constexpr (JAG) return launch_one<D, QH, kWavesJagged, true>(p, grid, stream);
  else if constexpr (D == 128)
    return dense_waves(D, p.causal && p.window > 0) == 4 ? launch_one<D, QH, 4, false>(p, grid, stream)
                                                          : launch_one<D, QH, 8, false>(p, grid, stream);
  else return launch_one<D, QH, kWavesDense, false>(p, grid, stream);
}

// JAG: the persistent instances of jagged batches (p.sched set), else the dense ones
template <int D, bool JAG>
inline hipError_t launch_qh(const PrefillParams& p, int qh, int grid, hipStream_t stream) {
  switch (qh) {
    case 1: return launch_nw<D, 1, JAG>(p, grid, stream);
    case 2: return launch_nw<D, 2, JAG>(p, grid, stream);
    case 4: return launch_nw<D, 4, JAG>(p, grid, stream);
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
