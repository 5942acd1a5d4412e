/*
 * fakv.h -- C ABI of the MI355X (gfx950) blockwise-attention library.
 *
 * What it computes: scaled-dot-product attention evaluated block by block.
 * Every key/value block yields a partial triplet (m, l, O) -- the row max of
 * the scaled scores, the row sum of exp(score - m), and exp(score - m) @ V
 * left unnormalised -- and triplets fold into a running state by the
 * online-softmax merge
 *     m' = max(m1, m2),  l' = l1 e^(m1-m') + l2 e^(m2-m'),  O' = O1 e^(m1-m') + O2 e^(m2-m'),
 * with the final output O / l.  Sources (web pages, by title and section):
 *   - "_gqa_prefill_long.py" (kernbench2 GQA fused-attention prefill with Ring
 *     KV): the step-0 partial, the ring steps with their merge, final O / l;
 *   - "[pallas] Support dependent Tile.end bounds in Pallas" (Helion): the
 *     causal inner loop ending at the smaller of the KV end and the query
 *     tile's end ("Bound recognition", "Unroll lowering") and flattened
 *     (sequence, query-tile) worklists ("Flattened worklists");
 *   - "_attention_mesh_mlo.py" (kernbench2 mesh-native mlo decode): the
 *     one-shot local partial of sequence-sharded decode and the merge of the
 *     per-rank triplets.
 *
 * Conventions shared by every entry point
 *   - Softmax scale is 1/sqrt(d).  m is exported in natural-log units of the
 *     scaled score.
 *   - Layouts are token-major and contiguous: Q and O are (tokens, h_q, d);
 *     K and V are (tokens, h_kv, d).  Query head h reads KV head h / (h_q/h_kv).
 *   - Causal: key position <= query position (top-left alignment).
 *   - dtype: FAKV_BF16 (inputs bf16, fp32 accumulation, output bf16 rounded to
 *     nearest even) or FAKV_F32 (fp32 throughout).  Triplets are always fp32.
 *   - d must be 64, 128 or 256.  Every device pointer must be 16-byte aligned.
 *   - Ownership: the caller owns every buffer, workspaces included.  The
 *     library never allocates, frees or synchronises on these paths; each call
 *     only enqueues kernels on `stream` (a hipStream_t; NULL = null stream)
 *     of the current HIP device, and returns.  A workspace holds a call's
 *     intermediate state (worklists, queue counters, partial triplets) until
 *     that call's kernels finish: calls that may run at the same time need
 *     distinct workspaces, while calls ordered on one stream may share one.
 *     Its contents on entry do not matter.
 *   - Errors: every argument check runs on the host before anything is
 *     enqueued.  An invalid argument returns FAKV_EINVAL, a valid but
 *     unsupported combination FAKV_EUNSUPPORTED; in both cases nothing is
 *     enqueued.  A failed kernel launch returns FAKV_EDEVICE.  fakv_last_error()
 *     describes the most recent failure on the calling thread.  No C++
 *     exception crosses this interface.
 *   - Determinism: fixed reduction orders, no floating-point atomics; the same
 *     call on the same inputs gives bitwise-identical outputs.
 */
#ifndef FAKV_H
#define FAKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FAKV_OK = 0,
  FAKV_EINVAL = 1,
  FAKV_EUNSUPPORTED = 2,
  FAKV_EDEVICE = 3
} fakv_status;

typedef enum { FAKV_F32 = 0, FAKV_BF16 = 1 } fakv_dtype;

/* Size in bytes of one worklist record: int32 x 8 =
 * (seq, tile, range_start, range_len, tile_start, tile_extent, compute_end, 0). */
#define FAKV_WORKITEM_BYTES 32

/*
 * attn_partial -- one block step of the prefill page's ring loop.
 *
 * Partial triplet of every query row of q (T_q, h_q, d) against one KV chunk
 * k, v (S_chunk, h_kv, d).  Query row i sits at position q_pos0 + i and key j
 * at k_pos0 + j; with causal != 0 a key is admissible iff its position is <=
 * the query's.  Within the chunk the key loop ends at the smaller of the chunk
 * end and the query tile's end (tiles past it are never visited).
 *   accumulate == 0: writes the chunk's triplet to m, l (T_q, h_q) and
 *                    o_acc (T_q, h_q, d), all fp32; a row with no admissible
 *                    key gets the identity (-inf, 0, 0).
 *   accumulate != 0: reads the running state from m, l, o_acc and writes back
 *                    its merge with the chunk's triplet (the prefill page's
 *                    online-softmax step); a row with no admissible key keeps
 *                    its state.
 * Preconditions: T_q >= 0, S_chunk >= 0, h_q % h_kv == 0, and every position
 * (q_pos0 .. q_pos0 + T_q, k_pos0 .. k_pos0 + S_chunk) within [-2^29, 2^29]
 * (else FAKV_EINVAL: the kernels compare positions in 32 bits).  T_q == 0 enqueues
 * nothing (the pointers may then be NULL); S_chunk == 0 writes identities
 * (accumulate == 0) or nothing, and k, v may then be NULL.
 */
fakv_status attn_partial(const void* q, const void* k, const void* v,
                         float* m, float* l, float* o_acc,
                         int T_q, int S_chunk, int h_q, int h_kv, int d,
                         int q_pos0, int k_pos0, int causal, int accumulate,
                         int dtype, void* stream);

/*
 * lse_merge -- fold n_parts triplets per row into the final output.
 *
 * m_parts, l_parts: (n_parts, rows) fp32; o_parts: (n_parts, rows, d) fp32
 * (unnormalised O).  Per row the online-softmax merge is applied to all parts
 * at once: the common max m' = max_c m_c first, then every part is rescaled by
 * exp(m_c - m') and the l's and O's are summed in a fixed order (a part with
 * m = -inf weighs 0), so results are reproducible.  Then O / l is written to
 * o_out (rows, d) in out_dtype, and
 * m + ln l to lse_out (rows) unless lse_out is NULL.  A row whose parts are
 * all empty (every m = -inf, l = 0) merges to the identity triplet: its output
 * row is written as zeros and its lse as -inf (the log of an empty sum).
 * This is the merge of the decode page's per-rank triplets and of the prefill
 * page's ring steps.  Preconditions: n_parts >= 1, rows >= 0.
 */
fakv_status lse_merge(const float* m_parts, const float* l_parts, const float* o_parts,
                      int n_parts, int rows, int d, void* o_out, float* lse_out,
                      int out_dtype, void* stream);

/*
 * ring_attn_fwd -- prefill attention, whole ring fused in one launch.
 *
 * seq_offsets == NULL: a dense batch of n_seqs sequences, each with T_q
 *   queries and S_kv keys; q is (n_seqs*T_q, h_q, d), k and v are
 *   (n_seqs*S_kv, h_kv, d), o is (n_seqs*T_q, h_q, d).  S_kv % C == 0.
 *   Causal requires T_q == S_kv.
 * seq_offsets != NULL: a jagged self-attention batch packed by device int32
 *   prefix offsets seq_offsets[0..n_seqs] (non-decreasing, seq_offsets[0] ==
 *   0, seq_offsets[n_seqs] == T_q); T_q == S_kv == total tokens.  Sequence b
 *   is split into C contiguous chunks of ceil(L_b / C) keys.  The offsets are
 *   read on the device only (no host synchronisation); a device-built
 *   (sequence, query-tile) worklist, longest tiles first, lives in the
 *   workspace.  Offsets that are not such a prefix array are detected on the
 *   device: the worklist comes out empty and o is left untouched (nothing is
 *   read or written out of bounds).
 * Each query tile takes the ring position of its first row, r = floor(i*C/L),
 * and visits KV chunks in the order (r + s) mod C, s = 0..C-1, as the prefill
 * page's rank r does after s westward rotations.  (A small fp32 dense call
 * instead computes the partial triplet of every chunk -- cut into equal parts
 * -- in separate workgroups and merges them in part order; see
 * ring_attn_workspace_bytes.)  Causal: a chunk starting at
 * or after the tile's end is skipped whole, and inside a chunk the key loop
 * ends at min(chunk end, query tile end) ("dependent Tile.end"), so only the
 * tiles straddling the diagonal apply an element mask.
 * workspace: at least ring_attn_workspace_bytes(...) bytes (may be NULL when
 * that is 0).  T_q == 0 (an empty dense batch, or a jagged batch whose
 * sequences are all empty) is a valid call that enqueues nothing; q, k, v, o
 * and workspace may then be NULL.
 */
fakv_status ring_attn_fwd(const void* q, const void* k, const void* v, void* o,
                          int T_q, int S_kv, int h_q, int h_kv, int d, int C, int causal,
                          const int32_t* seq_offsets, int n_seqs, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * ring_attn_fwd_window -- causal prefill restricted to a sliding window.
 *
 * As ring_attn_fwd with causal = 1, except that query i of a sequence sees
 * only keys i - window < j <= i (local positions): the dependent *lower*
 * bound that the Helion page ("Scalar minimum") leaves to sliding-window
 * support.  The KV walk of a query tile starts at the tile holding
 * max(chunk start, tile start - window + 1), chunks wholly below it are
 * skipped, and only tiles crossing either edge of the band are masked.
 * window >= the sequence length gives plain causal attention (a window longer
 * than every sequence is taken as the longest sequence's length).  Same layouts,
 * workspace and errors as ring_attn_fwd; window < 1 is FAKV_EINVAL.
 */
fakv_status ring_attn_fwd_window(const void* q, const void* k, const void* v, void* o,
                                 int T_q, int S_kv, int h_q, int h_kv, int d, int C, int window,
                                 const int32_t* seq_offsets, int n_seqs, int dtype,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace needed by ring_attn_fwd for these arguments (jagged = seq_offsets
 * != NULL).  Dense bf16 batches need none (0).  A dense fp32 call whose query
 * tiles would occupy few compute units is split over its KV range -- each
 * ring chunk cut into equal parts, one partial triplet per (query tile,
 * part), merged by the lse_merge kernel -- and needs room for those fp32
 * triplets; larger fp32 calls need none. */
size_t ring_attn_workspace_bytes(int T_q, int S_kv, int h_q, int h_kv, int d, int C,
                                 int causal, int n_seqs, int jagged, int dtype);

/*
 * splitkv_decode -- one decode step over a sequence-split KV cache.
 *
 * q (B, h_q, d): one query token per sequence.  k, v (B, S_kv, h_kv, d): the
 * cache.  Each sequence's keys are cut into n_chunks contiguous chunks of
 * ceil(S_kv / n_chunks) keys (the last chunks may be short or empty).  One
 * kernel computes every (sequence, KV head, chunk) local partial for all
 * h_q/h_kv query heads of the group at once (K and V are read from HBM once),
 * writing fp32 triplets into the workspace; a second kernel merges each
 * (sequence, query head)'s n_chunks triplets in a fixed tree and writes
 * o (B, h_q, d) in dtype.  This is the decode page's local partial per rank
 * followed by its (m, l, o) merge, with the ranks laid side by side on one GPU.
 * workspace: at least splitkv_decode_workspace_bytes(B, h_q, d, n_chunks).
 * Preconditions: dtype == FAKV_BF16, B >= 1, S_kv >= 1, 1 <= n_chunks <= S_kv,
 * h_q / h_kv <= 32 (the query heads of a group are the 32 columns of one
 * MFMA tile); otherwise FAKV_EINVAL / FAKV_EUNSUPPORTED and nothing enqueued.
 */
fakv_status splitkv_decode(const void* q, const void* k, const void* v, void* o,
                           int B, int h_q, int h_kv, int d, int S_kv, int n_chunks,
                           int dtype, void* workspace, size_t workspace_bytes, void* stream);

size_t splitkv_decode_workspace_bytes(int B, int h_q, int d, int n_chunks);

/* Bytes of device scratch the library itself holds per device for
 * splitkv_decode_noalloc (32 MiB). */
#define FAKV_DECODE_SCRATCH_BYTES (32u << 20)

/*
 * splitkv_decode_noalloc -- splitkv_decode without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * layouts, kernels, results and errors as splitkv_decode, except that the
 * partial triplets go to a scratch array the library holds on each device
 * (FAKV_DECODE_SCRATCH_BYTES, allocated with the library's code on that
 * device and kept until the process ends).  The call itself allocates and
 * frees nothing; its first call on a device looks up that device's scratch
 * address.  A call whose partials need more than the scratch
 * (splitkv_decode_workspace_bytes(B, h_q, d, n_chunks) >
 * FAKV_DECODE_SCRATCH_BYTES) returns FAKV_EINVAL and enqueues nothing.
 * Every call on one device shares that scratch, and every call overwrites
 * all of the triplets it reads: calls that may overlap on one device (on
 * different streams, or from several threads) race and must be serialised
 * by the caller, e.g. on one stream.
 */
fakv_status splitkv_decode_noalloc(const void* q, const void* k, const void* v, void* o,
                                   int B, int h_q, int h_kv, int d, int S_kv, int n_chunks,
                                   int dtype, void* stream);

/*
 * fakv_jagged_worklist -- build the flattened (sequence, query-tile) worklist
 * of a jagged batch on the device ("Flattened worklists" of the Helion page):
 * one FAKV_WORKITEM_BYTES record per tile of BQ query rows, with the resident
 * source range of its sequence, the tile's compact extent and compute_end =
 * min(source end, tile end); ordered by descending tile index, ties by
 * ascending sequence.  items must hold `capacity` records; the record count is
 * written to *n_items (device int32).  Returns FAKV_EINVAL if capacity is
 * below total_tokens / BQ + n_seqs (the bound that every valid offset array
 * respects).  ring_attn_fwd builds the same list internally.
 */
fakv_status fakv_jagged_worklist(const int32_t* seq_offsets, int n_seqs, int total_tokens,
                                 int BQ, int32_t* items, int32_t* n_items, size_t capacity,
                                 void* stream);

/* Query-tile height of the worklist ring_attn_fwd builds for a jagged batch
 * with these arguments (its BQ; bf16 dense batches run 4-wave tiles half as
 * tall, except d = 128 without a sliding window, which runs this height).
 * 0 for arguments ring_attn_fwd rejects (h_q not a multiple of h_kv, d). */
int fakv_query_tile_rows(int h_q, int h_kv, int d, int dtype);

/* Message describing the last failure on the calling thread ("" if none).
 * Valid until the next library call on that thread. */
const char* fakv_last_error(void);

/* ABI version of this header (major * 100 + minor): 102. */
int fakv_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FAKV_H */
