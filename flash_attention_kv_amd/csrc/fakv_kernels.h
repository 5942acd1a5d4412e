// fakv_kernels.h -- kernel parameter blocks and launchers (library-internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace fakv {

// Parameters of one prefill launch.  Dense batches (items == nullptr) have
// n_seqs sequences of T_q queries / S_kv keys; jagged batches read their
// (sequence, query tile) items from a device worklist.
struct PrefillParams {
  const uint16_t* q;       // bf16 bits, or fp32 via the f32 kernels' cast
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;             // mode 0: output in the input dtype
  float* m_st;             // modes 1, 2: triplet state (T, h_q)
  float* l_st;             //                            (T, h_q)
  float* o_st;             //                            (T, h_q, d)
  int mode;                // 0 = O / l, 1 = write triplet, 2 = merge into triplet
  int n_seqs, T_q, S_kv;
  int h_q, h_kv;
  int C, causal, prune;
  int q_pos0, k_pos0;
  const int32_t* items;    // jagged worklist records (8 x int32), or nullptr
  const int32_t* n_items;  // device count of records
  const int32_t* sched;    // bf16 jagged: 8 per-XCD queues of item * n_hg + head group
  int sched_stride;        // entries reserved per queue
  int32_t* qinfo;          // queue lengths [0..7]; the queues' pop counters at [16 + 4 q]
  int n_qtiles;            // dense: query tiles per sequence
  int n_hg;                // workgroups per query tile = h_q / heads per workgroup
  float scale;             // 1 / sqrt(d)
  float scale_log2;        // scale * log2(e)
  int window;              // causal sliding window in keys (query i sees i - window < j <= i); 0 = none
  int kv_parts;            // fp32 dense split-KV: workgroups per query tile, one KV part each
                           // (mode 1 triplets at part * rows); 0 = one workgroup walks the ring
};

struct DecodeParams {
  const uint16_t* q;       // (B, h_q, d) bf16
  const uint16_t* k;       // (B, S, h_kv, d)
  const uint16_t* v;
  float* m_parts;          // (n_chunks, B*h_q)
  float* l_parts;
  float* o_parts;          // (n_chunks, B*h_q, d)
  int B, h_q, h_kv, S, n_chunks, chunk_w;
  float scale, scale_log2;
};

struct MergeParams {
  const float* m_parts;
  const float* l_parts;
  const float* o_parts;
  int n_parts, rows;
  void* o_out;
  float* lse_out;
  int out_bf16;
};

// Per-device one-time raise of a kernel's dynamic-LDS limit.
hipError_t ensure_lds_limit(const void* fn, int bytes, std::atomic<unsigned>& done_mask);

// Query rows of one bf16 workgroup tile for head dim d and qh query heads
// per workgroup, for a dense or a jagged batch, with or without a window.
int prefill_bf16_query_rows(int d, int qh, bool jagged, bool window);
hipError_t launch_prefill_bf16(const PrefillParams& p, int d, int qh, int grid, hipStream_t stream);
// d = 256 instances (their own translation unit, see prefill_bf16_d256.hip)
hipError_t launch_prefill_bf16_d256(const PrefillParams& p, int qh, int grid, hipStream_t stream);
int prefill_bf16_resident_d256(int qh);
// jagged d = 64 and 128 instances (their own translation unit, see prefill_bf16_jagged.hip)
hipError_t launch_prefill_bf16_jagged(const PrefillParams& p, int d, int qh, int grid, hipStream_t stream);
int prefill_bf16_resident_jagged(int d, int qh);
hipError_t launch_prefill_f32(const PrefillParams& p, int d, int grid, hipStream_t stream);
constexpr int kF32QueryTile = 128;   // query rows per fp32 workgroup
hipError_t launch_decode_partial(const DecodeParams& p, int d, int g, hipStream_t stream);
hipError_t launch_lse_merge(const MergeParams& p, int d, hipStream_t stream);
hipError_t launch_worklist(const int32_t* seq_offsets, int n_seqs, int total, int BQ,
                           int32_t* items, int32_t* n_items, int capacity, hipStream_t stream);

// Workspace carve-up of the per-XCD schedule built after the worklist.
struct SchedBufs {
  int32_t* qinfo;          // queue lengths [0..7]; pop counters at [16 + 4 q] (the schedule kernel zeroes them)
  int32_t* nat2canon;      // capacity ints: (seq, tile) in natural order -> record index
  int32_t* ntprefix;       // n_seqs + 1 ints: prefix sums of tiles per sequence
  int32_t* seq_of_rank;    // n_seqs ints: sequences sorted by tile count, descending
  int32_t* sched;          // 8 * stride ints
  int stride;
};
hipError_t launch_schedule(const int32_t* seq_offsets, int n_seqs, int BQ, const int32_t* items,
                           const int32_t* n_items, int n_hg, const SchedBufs& sb, hipStream_t stream);
// launch_worklist and launch_schedule in one launch (the same records and
// queues), for batches of at most 2048 sequences and 12288 worklist slots:
// plan_fits() says whether a batch qualifies.
bool plan_fits(int n_seqs, size_t capacity);
hipError_t launch_plan(const int32_t* seq_offsets, int n_seqs, int total, int BQ, int32_t* items,
                       int32_t* n_items, int capacity, int n_hg, const SchedBufs& sb, hipStream_t stream);
// Resident workgroups of the bf16 prefill kernel on the current device (for persistent grids).
int prefill_bf16_persistent_grid(int d, int qh);

}  // namespace fakv
