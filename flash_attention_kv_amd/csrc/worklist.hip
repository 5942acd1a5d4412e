// worklist.hip -- device build of the flattened (sequence, query-tile) list.
//
// "[pallas] Support dependent Tile.end bounds in Pallas", "Flattened
// worklists": each item records the resident source range of its sequence
// (start, length) and its query tile's compact extent (start, extent); its
// compute end is min(source end, tile end) and alone drives the KV trip count.
// The sequence ends come from the prefix offsets in device memory, so the
// list is built on the device and the host never synchronises.
//
// Order: tiles with the larger index t (longer causal KV ranges) first, ties
// by ascending sequence -- a longest-first schedule for the prefill grid.
// One workgroup of 1024 threads: for t = T-1 .. 0 it ranks the sequences with
// more than t tiles by a block-wide prefix count (wave ballots + popcounts)
// and scatters their records.  Offsets that are not a valid prefix array
// (first != 0, a decreasing pair, last != total) yield an empty list, so a
// bad argument can never make the prefill kernel read out of bounds.  Each
// pair is validated by a direct compare, never by the sign of a difference:
// a difference of two arbitrary int32 values can wrap to a positive length.
// Once every pair is non-decreasing from 0 to total, all offsets lie in
// [0, total] and no length computed from them can wrap.
#include "fakv_device.h"
#include "fakv_kernels.h"

namespace fakv {

__global__ __launch_bounds__(1024)
void worklist_kernel(const int32_t* __restrict__ off, int n_seqs, int total, int BQ,
                     int32_t* __restrict__ items, int32_t* __restrict__ n_items, int capacity) {
  constexpr int kCache = 8192;         // lengths of the first sequences, kept in LDS
  __shared__ int s_wave[16];
  __shared__ int s_max;
  __shared__ int s_bad;
  __shared__ int s_len[kCache];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) { s_max = 0; s_bad = (off[0] != 0 || off[n_seqs] != total) ? 1 : 0; }
  __syncthreads();
  int local_max = 0, bad = 0;
  for (int b = tid; b < n_seqs; b += 1024) {
    const int a0 = off[b], a1 = off[b + 1];
    if (a1 < a0) bad = 1;
    // (only used when every pair is ordered, so then 0 <= L <= total)
    const int L = bad ? 0 : a1 - a0;
    if (b < kCache) s_len[b] = L;
    local_max = max(local_max, L / BQ + (L % BQ != 0));
  }
  // the ranking passes below revisit every sequence once per tile index:
  // lengths come from LDS, not from global offsets, on that path
  auto len = [&](int b) { return b < kCache ? s_len[b] : off[b + 1] - off[b]; };
  if (bad) atomicOr(&s_bad, 1);
  atomicMax(&s_max, local_max);
  __syncthreads();
  if (s_bad) {
    if (tid == 0) *n_items = 0;
    return;
  }
  const int T = s_max;
  int base = 0;
  for (int t = T - 1; t >= 0; --t) {
    for (int b0 = 0; b0 < n_seqs; b0 += 1024) {
      const int b = b0 + tid;
      int L = 0;
      if (b < n_seqs) L = len(b);
      const bool flag = b < n_seqs && L > t * BQ;
      const unsigned long long bal = __ballot(flag);
      const int below = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) s_wave[wave] = __popcll(bal);
      __syncthreads();
      int pre = 0, tot = 0;
      for (int w = 0; w < 16; ++w) {
        const int cnt = s_wave[w];
        pre += (w < wave) ? cnt : 0;
        tot += cnt;
      }
      if (flag) {
        const int pos = base + pre + below;
        if (pos < capacity) {
          const int start = off[b];
          const int ts = start + t * BQ;
          const int ext = min(BQ, L - t * BQ);
          int32_t* r = items + 8 * (size_t)pos;
          r[0] = b; r[1] = t; r[2] = start; r[3] = L;
          r[4] = ts; r[5] = ext; r[6] = min(start + L, ts + ext); r[7] = 0;
        }
      }
      base += tot;
      __syncthreads();
    }
  }
  if (tid == 0) *n_items = min(base, capacity);
}

// ---------------------------------------------------------------------------
// Per-XCD schedule of a jagged batch (bf16 prefill).  Units are
// (sequence, head group) pairs; sequences are ranked by tile count, longest
// first, and the units of that order are dealt round-robin onto 8 queues
// (unit k -> queue k mod 8).  A unit's entries -- its query tiles, longest
// first -- are contiguous in its queue, so the workgroups that take them run
// at the same time on one XCD and share that sequence's K/V in its L2.
// Entry = record index * n_hg + head group.  Runs after worklist_kernel on
// the same stream; an empty worklist gives empty queues.  The order among
// sequences of equal tile count is whatever the LDS atomics produce: it only
// decides which workgroup computes an item, never a result.

// Exclusive prefix sum over the 1024 threads of the block: wave scans with
// lane shuffles, then one pass over the 16 wave totals.  Returns the block
// total; uses two barriers.
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  int pre = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int c = s_wave[w];
    pre += (w < wave) ? c : 0;
    total += c;
  }
  __syncthreads();
  return pre + x - v;
}

// Exclusive prefix sum over the threads of each residue class tid mod 8
// (the 8 queues): lane shuffles by 8, 16, 32 inside a wave, then the earlier
// waves' per-class totals.  Returns the class total of the block in total.
__device__ __forceinline__ int block_exclusive_scan8(int v, int* s_w8, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, x8 = threadIdx.x & 7;
  int x = v;
#pragma unroll
  for (int d = 8; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane >= 56) s_w8[wave * 8 + x8] = x;
  __syncthreads();
  int pre = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int c = s_w8[w * 8 + x8];
    pre += (w < wave) ? c : 0;
    total += c;
  }
  __syncthreads();
  return pre + x - v;
}

__global__ __launch_bounds__(1024)
void schedule_kernel(const int32_t* __restrict__ off, int n_seqs, int BQ, const int32_t* __restrict__ items,
                     const int32_t* __restrict__ n_items_p, int n_hg, SchedBufs sb) {
  __shared__ int s_wave[16];
  __shared__ int s_w8[128];
  __shared__ int s_carry[8];
  __shared__ int s_max;
  __shared__ int s_hist[1025];         // tile counts 1 .. 1024 (larger ones share the last bin)
  const int tid = threadIdx.x;
  const int n_items = *n_items_p;
  if (n_items == 0) {          // empty batch or rejected offsets
    if (tid < 16) sb.qinfo[tid] = 0;
    if (tid < 8) sb.qinfo[16 + 4 * tid] = 0;        // the queues' pop counters
    return;
  }
  // (offsets are a valid prefix array here: worklist_kernel checked every
  // pair by direct compares, so 0 <= L <= total and L cannot wrap)
  auto ntiles = [&](int b) {
    const int L = off[b + 1] - off[b];
    return L / BQ + (L % BQ != 0);
  };
  auto bin = [&](int v) { return min(v, 1024); };

  // 1. exclusive prefix sums of tiles per sequence; histogram of tile counts
  for (int i = tid; i < 1025; i += 1024) s_hist[i] = 0;
  if (tid == 0) s_max = 0;
  __syncthreads();
  int carry = 0;
  for (int b0 = 0; b0 < n_seqs; b0 += 1024) {
    const int b = b0 + tid;
    const int v = b < n_seqs ? ntiles(b) : 0;
    int tot;
    const int ex = block_exclusive_scan(v, s_wave, tot);
    if (b < n_seqs) {
      sb.ntprefix[b] = carry + ex;
      if (v > 0) atomicAdd(&s_hist[bin(v)], 1);
    }
    carry += tot;
  }
  if (tid == 0) sb.ntprefix[n_seqs] = carry;
  __syncthreads();                     // prefix sums and histogram complete

  // 2. (sequence, tile) in natural order -> worklist record index
  for (int i = tid; i < n_items; i += 1024) {
    const int32_t* r = items + 8 * (size_t)i;
    sb.nat2canon[sb.ntprefix[r[0]] + r[1]] = i;
  }
  __syncthreads();

  // 3. rank sequences by tile count, descending: start of each bin from the
  //    top, then one slot per sequence by an atomic cursor in its bin.
  //    Counts beyond 1024 tiles share the top bin; within it they are
  //    ordered by a second, exact pass.
  {
    int v = 0;
    if (tid < 1024) v = s_hist[1024 - tid];        // bins from the top: 1024, 1023, .. 1
    int tot;
    const int ex = block_exclusive_scan(v, s_wave, tot);
    if (tid < 1024) s_hist[1024 - tid] = ex;      // now: first rank of the bin
    __syncthreads();
    for (int b0 = 0; b0 < n_seqs; b0 += 1024) {
      const int b = b0 + tid;
      if (b < n_seqs) {
        const int nt = ntiles(b);
        if (nt > 0) sb.seq_of_rank[atomicAdd(&s_hist[bin(nt)], 1)] = b;
      }
    }
    if (tid == 0) s_max = tot;                     // non-empty sequences
    __syncthreads();
  }
  const int n_ranked = s_max;
  // sequences with more than 1024 tiles: order the top bin exactly (rare)
  if (s_hist[1024] > 0) {
    // top bin occupies ranks [0, n_big); sort it by count, descending (one thread)
    if (tid == 0) {
      int n_big = 0;
      while (n_big < n_ranked && ntiles(sb.seq_of_rank[n_big]) >= 1024) ++n_big;
      for (int i = 1; i < n_big; ++i) {
        const int x = sb.seq_of_rank[i];
        const int vx = ntiles(x);
        int j = i - 1;
        while (j >= 0 && ntiles(sb.seq_of_rank[j]) < vx) { sb.seq_of_rank[j + 1] = sb.seq_of_rank[j]; --j; }
        sb.seq_of_rank[j + 1] = x;
      }
    }
  }
  __syncthreads();
  const int n_units = n_ranked * n_hg;   // non-empty sequences x head groups

  // 4. deal units onto the queues; per-queue offsets by a stride-8 scan
  if (tid < 8) s_carry[tid] = 0;
  __syncthreads();
  for (int k0 = 0; k0 < n_units; k0 += 1024) {
    const int k = k0 + tid;
    const bool valid = k < n_units;
    const int r = valid ? k / n_hg : 0;
    const int hg = valid ? k - r * n_hg : 0;
    const int b = valid ? sb.seq_of_rank[r] : 0;
    const int v = valid ? ntiles(b) : 0;
    const int x = tid & 7;             // == k mod 8 since k0 is a multiple of 1024
    int tot;
    const int ex = block_exclusive_scan8(v, s_w8, tot);
    if (valid) {
      const int pos = s_carry[x] + ex;
      int32_t* q = sb.sched + (size_t)x * sb.stride + pos;
      const int32_t* nc = sb.nat2canon + sb.ntprefix[b];
      for (int j = 0; j < v; ++j) q[j] = nc[v - 1 - j] * n_hg + hg;
    }
    __syncthreads();
    if (tid < 8) s_carry[tid] += tot;
    __syncthreads();
  }
  if (tid < 8) sb.qinfo[tid] = s_carry[tid];
  if (tid < 8) sb.qinfo[16 + 4 * tid] = 0;          // the queues' pop counters
}

// ---------------------------------------------------------------------------
// worklist_kernel and schedule_kernel fused into one launch, for batches whose
// per-sequence tables fit in LDS (kPlanSeqs sequences, kPlanItems worklist
// slots): the same records in the same order, and queues dealt by the same
// rule.  The sequence starts, tile counts, tile prefix sums, the ranking by
// tile count and the (sequence, tile) -> record map stay in LDS, so no pass
// waits on a global load, and each ranking pass takes one barrier (two
// alternating copies of the per-wave counts).
constexpr int kPlanSeqs = 2048;
constexpr int kPlanItems = 12288;

__global__ __launch_bounds__(1024)
void plan_kernel(const int32_t* __restrict__ off, int n_seqs, int total, int BQ, int32_t* __restrict__ items,
                 int32_t* __restrict__ n_items, int capacity, int n_hg, SchedBufs sb) {
  __shared__ int s_wave[2][16];
  __shared__ int s_w8[128];
  __shared__ int s_carry[8];
  __shared__ int s_max, s_bad, s_ranked;
  __shared__ int s_hist[1025];                 // tile counts 1 .. 1024 (larger ones share the last bin)
  __shared__ int s_start[kPlanSeqs];
  __shared__ int s_nt[kPlanSeqs];              // tiles per sequence
  __shared__ int s_pre[kPlanSeqs + 1];         // exclusive prefix sums of s_nt
  __shared__ int s_rank[kPlanSeqs];            // sequences by tile count, descending
  __shared__ int s_idx[kPlanItems];            // (sequence, tile) in natural order -> record index
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto bin = [&](int v) { return min(v, 1024); };

  // 1. validate the offsets (direct compares, as in worklist_kernel), lengths
  //    as tile counts, histogram and prefix sums of the counts
  for (int i = tid; i < 1025; i += 1024) s_hist[i] = 0;
  if (tid == 0) { s_max = 0; s_bad = (off[0] != 0 || off[n_seqs] != total) ? 1 : 0; }
  __syncthreads();
  int local_max = 0, bad = 0;
  for (int b = tid; b < n_seqs; b += 1024) {
    const int a0 = off[b], a1 = off[b + 1];
    if (a1 < a0) bad = 1;
    const int L = bad ? 0 : a1 - a0;
    const int nt = L / BQ + (L % BQ != 0);
    s_start[b] = a0;
    s_nt[b] = nt;
    local_max = max(local_max, nt);
  }
  if (bad) atomicOr(&s_bad, 1);
  atomicMax(&s_max, local_max);
  __syncthreads();
  if (s_bad) {                                 // rejected offsets: empty list, empty queues
    if (tid == 0) *n_items = 0;
    if (tid < 16) sb.qinfo[tid] = 0;
    if (tid < 8) sb.qinfo[16 + 4 * tid] = 0;
    return;
  }
  {
    int carry = 0;
    for (int b0 = 0; b0 < n_seqs; b0 += 1024) {
      const int b = b0 + tid;
      const int v = b < n_seqs ? s_nt[b] : 0;
      int tot;
      const int ex = block_exclusive_scan(v, s_wave[0], tot);
      if (b < n_seqs) {
        s_pre[b] = carry + ex;
        if (v > 0) atomicAdd(&s_hist[bin(v)], 1);
      }
      carry += tot;
    }
    if (tid == 0) s_pre[n_seqs] = carry;
  }
  __syncthreads();

  // 2. the worklist: tile index t = T-1 .. 0, sequences with more than t
  //    tiles in ascending order, ranked by wave ballots
  const int T = s_max;
  int base = 0, it = 0;
  for (int t = T - 1; t >= 0; --t) {
    for (int b0 = 0; b0 < n_seqs; b0 += 1024, ++it) {
      const int b = b0 + tid;
      const bool flag = b < n_seqs && s_nt[b] > t;
      const unsigned long long bal = __ballot(flag);
      const int below = __popcll(bal & ((1ull << lane) - 1ull));
      int* sw = s_wave[it & 1];
      if (lane == 0) sw[wave] = __popcll(bal);
      __syncthreads();
      int pre = 0, tot = 0;
      for (int w = 0; w < 16; ++w) {
        const int cnt = sw[w];
        pre += (w < wave) ? cnt : 0;
        tot += cnt;
      }
      if (flag) {
        const int pos = base + pre + below;
        if (pos < capacity) {
          const int start = s_start[b];
          const int L = (b + 1 < n_seqs ? s_start[b + 1] : total) - start;
          const int ts = start + t * BQ;
          const int ext = min(BQ, L - t * BQ);
          int32_t* r = items + 8 * (size_t)pos;
          r[0] = b; r[1] = t; r[2] = start; r[3] = L;
          r[4] = ts; r[5] = ext; r[6] = min(start + L, ts + ext); r[7] = 0;
          if (s_pre[b] + t < kPlanItems) s_idx[s_pre[b] + t] = pos;
        }
      }
      base += tot;
    }
  }
  if (tid == 0) *n_items = min(base, capacity);
  __syncthreads();                             // the last pass's reads of s_wave are done

  // 3. rank the sequences by tile count, descending (as schedule_kernel)
  {
    const int v = s_hist[1024 - tid];          // bins from the top: 1024, 1023, .. 1
    int tot;
    const int ex = block_exclusive_scan(v, s_wave[0], tot);
    s_hist[1024 - tid] = ex;                   // now: first rank of the bin
    __syncthreads();
    for (int b = tid; b < n_seqs; b += 1024) {
      const int nt = s_nt[b];
      if (nt > 0) s_rank[atomicAdd(&s_hist[bin(nt)], 1)] = b;
    }
    if (tid == 0) s_ranked = tot;              // non-empty sequences
    __syncthreads();
  }
  const int n_ranked = s_ranked;
  if (s_hist[1024] > 0 && tid == 0) {          // counts beyond 1024 tiles: order the top bin exactly
    int n_big = 0;
    while (n_big < n_ranked && s_nt[s_rank[n_big]] >= 1024) ++n_big;
    for (int i = 1; i < n_big; ++i) {
      const int x = s_rank[i];
      const int vx = s_nt[x];
      int j = i - 1;
      while (j >= 0 && s_nt[s_rank[j]] < vx) { s_rank[j + 1] = s_rank[j]; --j; }
      s_rank[j + 1] = x;
    }
  }
  if (tid < 8) s_carry[tid] = 0;
  __syncthreads();

  // 4. deal the units (sequence, head group) round-robin onto the 8 queues
  const int n_units = n_ranked * n_hg;
  for (int k0 = 0; k0 < n_units; k0 += 1024) {
    const int k = k0 + tid;
    const bool valid = k < n_units;
    const int r = valid ? k / n_hg : 0;
    const int hg = valid ? k - r * n_hg : 0;
    const int b = valid ? s_rank[r] : 0;
    const int v = valid ? s_nt[b] : 0;
    const int x = tid & 7;                     // == k mod 8 since k0 is a multiple of 1024
    int tot;
    const int ex = block_exclusive_scan8(v, s_w8, tot);
    if (valid) {
      int32_t* q = sb.sched + (size_t)x * sb.stride + s_carry[x] + ex;
      const int* nc = s_idx + s_pre[b];
      for (int j = 0; j < v; ++j) q[j] = nc[v - 1 - j] * n_hg + hg;
    }
    __syncthreads();
    if (tid < 8) s_carry[tid] += tot;
    __syncthreads();
  }
  if (tid < 8) sb.qinfo[tid] = s_carry[tid];
  if (tid < 8) sb.qinfo[16 + 4 * tid] = 0;     // the queues' pop counters
}

bool plan_fits(int n_seqs, size_t capacity) {
  return n_seqs <= kPlanSeqs && capacity <= (size_t)kPlanItems;
}

hipError_t launch_plan(const int32_t* seq_offsets, int n_seqs, int total, int BQ, int32_t* items,
                       int32_t* n_items, int capacity, int n_hg, const SchedBufs& sb, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, seq_offsets, n_seqs, total, BQ, items,
                     n_items, capacity, n_hg, sb);
  return hipGetLastError();
}

hipError_t launch_schedule(const int32_t* seq_offsets, int n_seqs, int BQ, const int32_t* items,
                           const int32_t* n_items, int n_hg, const SchedBufs& sb, hipStream_t stream) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(1024), 0, stream, seq_offsets, n_seqs, BQ, items,
                     n_items, n_hg, sb);
  return hipGetLastError();
}

hipError_t launch_worklist(const int32_t* seq_offsets, int n_seqs, int total, int BQ,
                           int32_t* items, int32_t* n_items, int capacity, hipStream_t stream) {
  hipLaunchKernelGGL(worklist_kernel, dim3(1), dim3(1024), 0, stream, seq_offsets, n_seqs, total,
                     BQ, items, n_items, capacity);
  return hipGetLastError();
}

}  // namespace fakv
