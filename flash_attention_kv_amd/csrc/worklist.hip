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
// (first != 0, decreasing, last != total) yield an empty list, so a bad
// argument can never make the prefill kernel read out of bounds.
#include "fakv_device.h"
#include "fakv_kernels.h"

namespace fakv {

__global__ __launch_bounds__(1024)
void worklist_kernel(const int32_t* __restrict__ off, int n_seqs, int total, int BQ,
                     int32_t* __restrict__ items, int32_t* __restrict__ n_items, int capacity) {
  __shared__ int s_wave[16];
  __shared__ int s_max;
  __shared__ int s_bad;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) { s_max = 0; s_bad = (off[0] != 0 || off[n_seqs] != total) ? 1 : 0; }
  __syncthreads();
  int local_max = 0, bad = 0;
  for (int b = tid; b < n_seqs; b += 1024) {
    const int L = off[b + 1] - off[b];
    if (L < 0) bad = 1;
    local_max = max(local_max, (max(L, 0) + BQ - 1) / BQ);
  }
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
      if (b < n_seqs) L = off[b + 1] - off[b];
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

hipError_t launch_worklist(const int32_t* seq_offsets, int n_seqs, int total, int BQ,
                           int32_t* items, int32_t* n_items, int capacity, hipStream_t stream) {
  hipLaunchKernelGGL(worklist_kernel, dim3(1), dim3(1024), 0, stream, seq_offsets, n_seqs, total,
                     BQ, items, n_items, capacity);
  return hipGetLastError();
}

}  // namespace fakv
