// api.hip -- host side of the C ABI declared in include/fakv.h.
//
// Every entry point validates all arguments on the host before it makes any
// HIP call, so a rejected call enqueues nothing and needs no device.  Valid
// calls only enqueue kernels on the caller's stream: no allocation, no
// synchronisation.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "fakv.h"
#include "fakv_kernels.h"

namespace {

thread_local std::string g_err;

fakv_status fail(fakv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

fakv_status device_fail(const char* what, hipError_t e) {
  return fail(FAKV_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool supported_d(int d) { return d == 64 || d == 128 || d == 256; }

// Query heads sharing one KV tile per bf16 workgroup (a divisor of the GQA group, at most 4).
int heads_per_wg(int h_q, int h_kv) {
  const int g = h_q / h_kv;
  return (g % 4 == 0) ? 4 : (g % 2 == 0) ? 2 : 1;
}

// Query rows per workgroup tile; bf16 jagged batches, and dense d = 128 ones
// without a sliding window, use taller tiles (more waves share each K/V tile
// in LDS).
int query_tile(int h_q, int h_kv, int d, int dtype, bool jagged, bool window = false) {
  if (dtype == FAKV_F32) return fakv::kF32QueryTile;
  return fakv::prefill_bf16_query_rows(d, heads_per_wg(h_q, h_kv), jagged, window);
}

bool env_no_prune() {
  // Test hook: visit every tile of every chunk and rely on the element mask
  // alone (causal pruning must not change a single bit of the result).
  const char* s = std::getenv("FAKV_NO_PRUNE");
  return s != nullptr && s[0] == '1';
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t worklist_capacity(int total, int n_seqs, int BQ) {
  return (size_t)(total / BQ) + (size_t)n_seqs;
}

// Split-KV parts of an fp32 dense call (0 = one workgroup per query tile
// walks the whole ring).  When the query tiles alone would occupy few CUs,
// each ring chunk is cut into `sub` equal parts of at least one 32-key tile,
// sub dividing the chunk width, enough to give ~256 workgroups in all.
int f32_kv_parts(int T_q, int S_kv, int h_q, int n_seqs, int C) {
  const long long grid = (long long)((T_q + fakv::kF32QueryTile - 1) / fakv::kF32QueryTile) * h_q * n_seqs;
  if (grid >= 128 || C < 1 || S_kv % C) return 0;
  const int w = S_kv / C;
  const long long want = (256 + grid * C - 1) / (grid * C);
  int sub = 1;
  for (int t = 2; t <= w / 32 && t <= want; ++t)
    if (w % t == 0) sub = t;
  return C * sub > 1 ? C * sub : 0;
}

// fp32 split-KV workspace: [O parts][m parts][l parts].
size_t f32_split_bytes(int parts, size_t rows, int d) {
  const size_t n = (size_t)parts * rows;
  return align256(n * d * 4) + 2 * align256(n * 4);
}

// Jagged-batch workspace: [header 256 B: n_items; queue lengths and pop counters from byte 64] [records]
// and, for bf16, the per-XCD schedule arrays.
struct JaggedLayout {
  size_t items, nat2canon, ntprefix, seq_of_rank, sched, total;
  size_t cap, stride;
};
JaggedLayout jagged_layout(int T_q, int n_seqs, int BQ, int n_hg, bool sched) {
  JaggedLayout L{};
  L.cap = worklist_capacity(T_q, n_seqs, BQ);
  L.items = 256;
  size_t o = L.items + align256(L.cap * FAKV_WORKITEM_BYTES);
  if (sched) {
    L.stride = L.cap * (size_t)n_hg;
    L.nat2canon = o;   o += align256(L.cap * 4);
    L.ntprefix = o;    o += align256(((size_t)n_seqs + 1) * 4);
    L.seq_of_rank = o; o += align256((size_t)n_seqs * 4);
    L.sched = o;       o += align256(8 * L.stride * 4);
  }
  L.total = o;
  return L;
}

// empty: the call has no query rows, so no tensor is read and null pointers
// are accepted.
fakv_status check_prefill_common(const void* q, const void* k, const void* v, int h_q, int h_kv,
                                 int d, int dtype, bool empty = false, bool no_keys = false) {
  if ((!q || !k || !v) && !empty && !(no_keys && q))
    return fail(FAKV_EINVAL, "q, k and v must be non-null");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(FAKV_EINVAL, "q, k and v must be 16-byte aligned");
  if (h_q < 1 || h_kv < 1) return fail(FAKV_EINVAL, "h_q and h_kv must be >= 1 (got %d, %d)", h_q, h_kv);
  if (h_q % h_kv) return fail(FAKV_EINVAL, "h_q (%d) must be a multiple of h_kv (%d)", h_q, h_kv);
  if (!supported_d(d)) return fail(FAKV_EUNSUPPORTED, "d = %d is not supported (64, 128, 256)", d);
  if (dtype != FAKV_F32 && dtype != FAKV_BF16) return fail(FAKV_EINVAL, "unknown dtype %d", dtype);
  return FAKV_OK;
}

// The bf16 prefill kernel addresses one (sequence, KV head)'s keys through a
// buffer resource with 32-bit byte offsets.
fakv_status check_kv_extent(long long keys, int h_kv, int d, int dtype) {
  if (dtype == FAKV_BF16 && keys * h_kv * d * 2 >= (1ll << 31))
    return fail(FAKV_EUNSUPPORTED, "one sequence's K/V span (%lld keys x %d heads x %d) exceeds 2 GiB", keys, h_kv, d);
  return FAKV_OK;
}

fakv::PrefillParams base_params(const void* q, const void* k, const void* v, int h_q, int h_kv,
                                int d) {
  fakv::PrefillParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.h_q = h_q;
  p.h_kv = h_kv;
  p.scale = 1.0f / std::sqrt((float)d);
  p.scale_log2 = p.scale * 1.4426950408889634f;
  p.prune = env_no_prune() ? 0 : 1;
  return p;
}

fakv_status launch_prefill(const fakv::PrefillParams& p, int d, int dtype, int grid, hipStream_t st) {
  hipError_t e;
  if (dtype == FAKV_BF16)
    e = fakv::launch_prefill_bf16(p, d, heads_per_wg(p.h_q, p.h_kv), grid, st);
  else
    e = fakv::launch_prefill_f32(p, d, grid, st);
  if (e != hipSuccess) return device_fail("prefill launch", e);
  return FAKV_OK;
}

}  // namespace

namespace fakv {

hipError_t ensure_lds_limit(const void* fn, int bytes, std::atomic<unsigned>& done_mask) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned bit = 1u << (dev & 31);
  if (done_mask.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  done_mask.fetch_or(bit, std::memory_order_acq_rel);
  return hipSuccess;
}

}  // namespace fakv

static fakv_status ring_attn_impl(const void* q, const void* k, const void* v, void* o, int T_q, int S_kv,
                                  int h_q, int h_kv, int d, int C, int causal, int window,
                                  const int32_t* seq_offsets, int n_seqs, int dtype, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  fakv_status s = check_prefill_common(q, k, v, h_q, h_kv, d, dtype, T_q == 0);
  if (s != FAKV_OK) return s;
  if (!o && T_q != 0) return fail(FAKV_EINVAL, "o must be non-null");
  if (!aligned16(o)) return fail(FAKV_EINVAL, "o must be 16-byte aligned");
  if (T_q < 0 || S_kv < 0) return fail(FAKV_EINVAL, "T_q and S_kv must be >= 0");
  if (C < 1) return fail(FAKV_EINVAL, "C must be >= 1 (got %d)", C);
  if (n_seqs < 0 || (seq_offsets == nullptr && n_seqs < 1))
    return fail(FAKV_EINVAL, "n_seqs must be >= 1 for a dense batch (got %d)", n_seqs);
  // A window as long as the longest sequence already admits every causal key;
  // longer ones are clamped to that, so no window bound on the device (query
  // position - window - key offset, in 32 bits) can wrap.
  const int longest = T_q > S_kv ? T_q : S_kv;
  if (window > longest) window = longest;
  const bool jagged = seq_offsets != nullptr;
  const int BQ = query_tile(h_q, h_kv, d, dtype, jagged, causal && window > 0);
  const int qh = dtype == FAKV_BF16 ? heads_per_wg(h_q, h_kv) : 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!jagged) {
    if (S_kv % C) return fail(FAKV_EINVAL, "S_kv (%d) must be a multiple of C (%d)", S_kv, C);
    if (causal && T_q != S_kv) return fail(FAKV_EINVAL, "causal attention needs T_q == S_kv (got %d, %d)", T_q, S_kv);
    if (T_q > 0 && S_kv == 0) return fail(FAKV_EINVAL, "queries without keys: attention is undefined");
    if ((long long)n_seqs * T_q * h_q * d >= (1ll << 40) || (long long)n_seqs * S_kv * h_kv * d >= (1ll << 40))
      return fail(FAKV_EINVAL, "tensor too large");
    if ((long long)n_seqs * T_q >= (1ll << 31) || (long long)n_seqs * S_kv >= (1ll << 31))
      return fail(FAKV_EINVAL, "token count exceeds int32");
    if ((s = check_kv_extent(S_kv, h_kv, d, dtype)) != FAKV_OK) return s;
    if (T_q == 0) return FAKV_OK;
    const int parts = dtype == FAKV_F32 ? f32_kv_parts(T_q, S_kv, h_q, n_seqs, C) : 0;
    const size_t rows = (size_t)n_seqs * T_q * h_q;
    if (parts > 0) {
      const size_t need = f32_split_bytes(parts, rows, d);
      if (workspace == nullptr || workspace_bytes < need)
        return fail(FAKV_EINVAL, "workspace too small: need %zu bytes, got %zu", need, workspace_bytes);
      if (!aligned16(workspace)) return fail(FAKV_EINVAL, "workspace must be 16-byte aligned");
    }
    fakv::PrefillParams p = base_params(q, k, v, h_q, h_kv, d);
    p.o = static_cast<uint16_t*>(o);
    p.mode = 0;
    p.n_seqs = n_seqs; p.T_q = T_q; p.S_kv = S_kv;
    p.C = C; p.causal = causal ? 1 : 0;
    p.window = window;
    p.n_qtiles = (T_q + BQ - 1) / BQ;
    p.n_hg = h_q / qh;
    const long long grid = (long long)p.n_qtiles * p.n_hg * n_seqs * (parts > 0 ? parts : 1);
    if (grid > 0x7fffffffll) return fail(FAKV_EINVAL, "grid too large");
    if (parts == 0) return launch_prefill(p, d, dtype, (int)grid, st);
    // fp32 split-KV: one partial triplet per (query tile, part), then the merge
    char* ws = static_cast<char*>(workspace);
    const size_t n = (size_t)parts * rows;
    p.mode = 1;
    p.kv_parts = parts;
    p.o_st = reinterpret_cast<float*>(ws);
    p.m_st = reinterpret_cast<float*>(ws + align256(n * d * 4));
    p.l_st = reinterpret_cast<float*>(ws + align256(n * d * 4) + align256(n * 4));
    if ((s = launch_prefill(p, d, dtype, (int)grid, st)) != FAKV_OK) return s;
    if (rows > 0x7fffffffull) return fail(FAKV_EINVAL, "too many rows");
    fakv::MergeParams mp{p.m_st, p.l_st, p.o_st, parts, (int)rows, o, nullptr, 0};
    hipError_t e = fakv::launch_lse_merge(mp, d, st);
    if (e != hipSuccess) return device_fail("split-KV merge launch", e);
    return FAKV_OK;
  }
  // jagged batch
  if (T_q != S_kv) return fail(FAKV_EINVAL, "a jagged batch needs T_q == S_kv == total tokens");
  if (n_seqs < 1) return fail(FAKV_EINVAL, "a jagged batch needs n_seqs >= 1");
  if (reinterpret_cast<uintptr_t>(seq_offsets) & 3u)
    return fail(FAKV_EINVAL, "seq_offsets must be 4-byte aligned");
  if ((long long)T_q * h_q * d >= (1ll << 40)) return fail(FAKV_EINVAL, "tensor too large");
  if ((s = check_kv_extent(S_kv, h_kv, d, dtype)) != FAKV_OK) return s;
  if (T_q == 0) return FAKV_OK;              // every sequence empty: no workspace, nothing to do
  const size_t need = ring_attn_workspace_bytes(T_q, S_kv, h_q, h_kv, d, C, causal, n_seqs, 1, dtype);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(FAKV_EINVAL, "workspace too small: need %zu bytes, got %zu", need, workspace_bytes);
  if (!aligned16(workspace)) return fail(FAKV_EINVAL, "workspace must be 16-byte aligned");
  const bool bf16 = dtype == FAKV_BF16;
  const int n_hg = h_q / qh;
  const JaggedLayout L = jagged_layout(T_q, n_seqs, BQ, n_hg, bf16);
  const size_t cap = L.cap;
  if (cap > 0x7fffffffull || (long long)cap * n_hg > 0x7fffffffll) return fail(FAKV_EINVAL, "grid too large");
  char* ws = static_cast<char*>(workspace);
  int32_t* n_items = reinterpret_cast<int32_t*>(ws);
  int32_t* items = reinterpret_cast<int32_t*>(ws + L.items);
  // bf16 batches whose tables fit build the worklist and the queues in one launch
  const bool plan = bf16 && fakv::plan_fits(n_seqs, cap);
  hipError_t e = hipSuccess;
  if (!plan) {
    e = fakv::launch_worklist(seq_offsets, n_seqs, T_q, BQ, items, n_items, (int)cap, st);
    if (e != hipSuccess) return device_fail("worklist launch", e);
  }
  fakv::PrefillParams p = base_params(q, k, v, h_q, h_kv, d);
  p.o = static_cast<uint16_t*>(o);
  p.mode = 0;
  p.n_seqs = n_seqs; p.T_q = T_q; p.S_kv = S_kv;
  p.C = C; p.causal = causal ? 1 : 0;
  p.window = window;
  p.items = items; p.n_items = n_items;
  p.n_hg = n_hg;
  if (!bf16) return launch_prefill(p, d, dtype, (int)(cap * n_hg), st);
  fakv::SchedBufs sb;
  sb.qinfo = reinterpret_cast<int32_t*>(ws + 64);
  sb.nat2canon = reinterpret_cast<int32_t*>(ws + L.nat2canon);
  sb.ntprefix = reinterpret_cast<int32_t*>(ws + L.ntprefix);
  sb.seq_of_rank = reinterpret_cast<int32_t*>(ws + L.seq_of_rank);
  sb.sched = reinterpret_cast<int32_t*>(ws + L.sched);
  sb.stride = (int)L.stride;
  if (plan) {
    e = fakv::launch_plan(seq_offsets, n_seqs, T_q, BQ, items, n_items, (int)cap, n_hg, sb, st);
    if (e != hipSuccess) return device_fail("plan launch", e);
  } else {
    e = fakv::launch_schedule(seq_offsets, n_seqs, BQ, items, n_items, n_hg, sb, st);
    if (e != hipSuccess) return device_fail("schedule launch", e);
  }
  p.sched = sb.sched;
  p.sched_stride = sb.stride;
  p.qinfo = sb.qinfo;
  return launch_prefill(p, d, dtype, fakv::prefill_bf16_persistent_grid(d, qh), st);
}

// ---------------------------------------------------------------------------
// Library-owned scratch of splitkv_decode_noalloc: the decode partial
// triplets live in this device array instead of a caller workspace.  Each
// device that runs the library holds its own copy (FAKV_DECODE_SCRATCH_BYTES)
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory, so host code never uses it directly: the device address
// of each device's copy is looked up once, with that device current, and kept
// in g_scratch_ptr[device].
static __device__ __align__(256) char scratch[FAKV_DECODE_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on first use).
fakv_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_fail("hipGetDevice", e);
  if (dev < 0 || dev >= kMaxDevices) return fail(FAKV_EUNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) return device_fail("hipGetSymbolAddress(scratch)", e);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FAKV_OK;
}
}  // namespace

extern "C" {

int fakv_abi_version(void) { return 102; }

const char* fakv_last_error(void) { return g_err.c_str(); }

int fakv_query_tile_rows(int h_q, int h_kv, int d, int dtype) {
  if (h_q < 1 || h_kv < 1 || h_q % h_kv || !supported_d(d)) return 0;
  return query_tile(h_q, h_kv, d, dtype, true);
}

size_t ring_attn_workspace_bytes(int T_q, int S_kv, int h_q, int h_kv, int d, int C, int causal,
                                 int n_seqs, int jagged, int dtype) {
  (void)causal;
  if (T_q <= 0 || n_seqs < 1 || h_q < 1 || h_kv < 1 || h_q % h_kv || !supported_d(d)) return 0;
  if (!jagged) {
    const int parts = dtype == FAKV_F32 ? f32_kv_parts(T_q, S_kv, h_q, n_seqs, C) : 0;
    return parts > 0 ? f32_split_bytes(parts, (size_t)n_seqs * T_q * h_q, d) : 0;
  }
  const int BQ = query_tile(h_q, h_kv, d, dtype, true);
  const bool bf16 = dtype == FAKV_BF16;
  const int n_hg = bf16 ? h_q / heads_per_wg(h_q, h_kv) : h_q;
  return jagged_layout(T_q, n_seqs, BQ, n_hg, bf16).total;
}

size_t splitkv_decode_workspace_bytes(int B, int h_q, int d, int n_chunks) {
  if (B < 1 || h_q < 1 || d < 1 || n_chunks < 1) return 0;
  const size_t parts = (size_t)n_chunks * B * h_q;
  return align256(parts * d * 4) + 2 * align256(parts * 4);
}

fakv_status attn_partial(const void* q, const void* k, const void* v, float* m, float* l,
                         float* o_acc, int T_q, int S_chunk, int h_q, int h_kv, int d, int q_pos0,
                         int k_pos0, int causal, int accumulate, int dtype, void* stream) {
  g_err.clear();
  // an empty chunk (S_chunk == 0) reads no key: k and v may then be NULL
  fakv_status s = check_prefill_common(q, k, v, h_q, h_kv, d, dtype, T_q == 0, S_chunk == 0);
  if (s != FAKV_OK) return s;
  if ((!m || !l || !o_acc) && T_q != 0) return fail(FAKV_EINVAL, "m, l and o_acc must be non-null");
  if (!aligned16(o_acc) || !aligned16(m) || !aligned16(l))
    return fail(FAKV_EINVAL, "m, l and o_acc must be 16-byte aligned");
  if (T_q < 0 || S_chunk < 0) return fail(FAKV_EINVAL, "T_q and S_chunk must be >= 0");
  // the kernels compare query and key positions in 32-bit arithmetic
  // (q_pos0 - k_pos0 plus a row or key index): keep every position within 2^29
  constexpr long long kPosLimit = 1ll << 29;
  if (q_pos0 < -kPosLimit || k_pos0 < -kPosLimit || (long long)q_pos0 + T_q > kPosLimit ||
      (long long)k_pos0 + S_chunk > kPosLimit)
    return fail(FAKV_EINVAL, "positions must lie within [-2^29, 2^29] (q_pos0 %d, k_pos0 %d)", q_pos0, k_pos0);
  if ((long long)T_q * h_q * d >= (1ll << 40) || (long long)S_chunk * h_kv * d >= (1ll << 40))
    return fail(FAKV_EINVAL, "tensor too large");
  if ((s = check_kv_extent(S_chunk, h_kv, d, dtype)) != FAKV_OK) return s;
  if (T_q == 0 || (S_chunk == 0 && accumulate)) return FAKV_OK;
  fakv::PrefillParams p = base_params(q, k, v, h_q, h_kv, d);
  p.m_st = m; p.l_st = l; p.o_st = o_acc;
  p.mode = accumulate ? 2 : 1;
  p.n_seqs = 1; p.T_q = T_q; p.S_kv = S_chunk;
  p.C = 1; p.causal = causal ? 1 : 0;
  p.q_pos0 = q_pos0; p.k_pos0 = k_pos0;
  const int BQ = query_tile(h_q, h_kv, d, dtype, false);
  const int qh = dtype == FAKV_BF16 ? heads_per_wg(h_q, h_kv) : 1;
  p.n_qtiles = (T_q + BQ - 1) / BQ;
  p.n_hg = h_q / qh;
  const long long grid = (long long)p.n_qtiles * p.n_hg;
  if (grid > 0x7fffffffll) return fail(FAKV_EINVAL, "grid too large");
  return launch_prefill(p, d, dtype, (int)grid, static_cast<hipStream_t>(stream));
}

fakv_status lse_merge(const float* m_parts, const float* l_parts, const float* o_parts, int n_parts,
                      int rows, int d, void* o_out, float* lse_out, int out_dtype, void* stream) {
  g_err.clear();
  if (!m_parts || !l_parts || !o_parts || !o_out)
    return fail(FAKV_EINVAL, "m_parts, l_parts, o_parts and o_out must be non-null");
  if (!aligned16(o_parts) || !aligned16(o_out)) return fail(FAKV_EINVAL, "o_parts and o_out must be 16-byte aligned");
  if (n_parts < 1 || rows < 0) return fail(FAKV_EINVAL, "need n_parts >= 1 and rows >= 0");
  if (!supported_d(d)) return fail(FAKV_EUNSUPPORTED, "d = %d is not supported (64, 128, 256)", d);
  if (out_dtype != FAKV_F32 && out_dtype != FAKV_BF16) return fail(FAKV_EINVAL, "unknown dtype %d", out_dtype);
  if (rows == 0) return FAKV_OK;
  fakv::MergeParams p{m_parts, l_parts, o_parts, n_parts, rows, o_out, lse_out, out_dtype == FAKV_BF16};
  hipError_t e = fakv::launch_lse_merge(p, d, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail("lse_merge launch", e);
  return FAKV_OK;
}

fakv_status ring_attn_fwd(const void* q, const void* k, const void* v, void* o, int T_q, int S_kv,
                          int h_q, int h_kv, int d, int C, int causal, const int32_t* seq_offsets,
                          int n_seqs, int dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
  g_err.clear();
  return ring_attn_impl(q, k, v, o, T_q, S_kv, h_q, h_kv, d, C, causal, 0, seq_offsets, n_seqs, dtype,
                        workspace, workspace_bytes, stream);
}

fakv_status ring_attn_fwd_window(const void* q, const void* k, const void* v, void* o, int T_q, int S_kv,
                                 int h_q, int h_kv, int d, int C, int window, const int32_t* seq_offsets,
                                 int n_seqs, int dtype, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  g_err.clear();
  if (window < 1) return fail(FAKV_EINVAL, "window must be >= 1 (got %d)", window);
  return ring_attn_impl(q, k, v, o, T_q, S_kv, h_q, h_kv, d, C, 1, window, seq_offsets, n_seqs, dtype,
                        workspace, workspace_bytes, stream);
}

}  // extern "C"

// Argument checks shared by splitkv_decode and splitkv_decode_noalloc.
static fakv_status check_decode(const void* q, const void* k, const void* v, void* o, int B, int h_q,
                                int h_kv, int d, int S_kv, int n_chunks, int dtype) {
  fakv_status s = check_prefill_common(q, k, v, h_q, h_kv, d, dtype);
  if (s != FAKV_OK) return s;
  if (!o) return fail(FAKV_EINVAL, "o must be non-null");
  if (!aligned16(o)) return fail(FAKV_EINVAL, "o must be 16-byte aligned");
  if (dtype != FAKV_BF16) return fail(FAKV_EUNSUPPORTED, "split-KV decode supports bf16 only");
  if (B < 1 || S_kv < 1) return fail(FAKV_EINVAL, "need B >= 1 and S_kv >= 1 (got %d, %d)", B, S_kv);
  if (n_chunks < 1 || n_chunks > S_kv)
    return fail(FAKV_EINVAL, "need 1 <= n_chunks <= S_kv (got %d)", n_chunks);
  if (h_q / h_kv > 32) return fail(FAKV_EUNSUPPORTED, "GQA group h_q/h_kv = %d exceeds 32", h_q / h_kv);
  if ((long long)B * S_kv * h_kv * d >= (1ll << 40)) return fail(FAKV_EINVAL, "tensor too large");
  if ((long long)B * h_q >= (1ll << 31)) return fail(FAKV_EINVAL, "B * h_q exceeds int32");
  if ((s = check_kv_extent(S_kv, h_kv, d, dtype)) != FAKV_OK) return s;
  if ((long long)B * h_kv * n_chunks > 0x7fffffffll) return fail(FAKV_EINVAL, "grid too large");
  return FAKV_OK;
}

// Enqueues the partial and merge kernels of a checked decode call; the
// partial triplets go to ws (at least splitkv_decode_workspace_bytes bytes).
static fakv_status enqueue_decode(const void* q, const void* k, const void* v, void* o, int B, int h_q,
                                  int h_kv, int d, int S_kv, int n_chunks, char* ws, void* stream) {
  const size_t parts = (size_t)n_chunks * B * h_q;
  fakv::DecodeParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o_parts = reinterpret_cast<float*>(ws);
  p.m_parts = reinterpret_cast<float*>(ws + align256(parts * d * 4));
  p.l_parts = reinterpret_cast<float*>(ws + align256(parts * d * 4) + align256(parts * 4));
  p.B = B; p.h_q = h_q; p.h_kv = h_kv; p.S = S_kv; p.n_chunks = n_chunks;
  p.chunk_w = (S_kv + n_chunks - 1) / n_chunks;
  p.scale = 1.0f / std::sqrt((float)d);
  p.scale_log2 = p.scale * 1.4426950408889634f;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = fakv::launch_decode_partial(p, d, h_q / h_kv, st);
  if (e != hipSuccess) return device_fail("decode partial launch", e);
  fakv::MergeParams mp{p.m_parts, p.l_parts, p.o_parts, n_chunks, B * h_q, o, nullptr, 1};
  e = fakv::launch_lse_merge(mp, d, st);
  if (e != hipSuccess) return device_fail("decode merge launch", e);
  return FAKV_OK;
}

extern "C" {

fakv_status splitkv_decode(const void* q, const void* k, const void* v, void* o, int B, int h_q,
                           int h_kv, int d, int S_kv, int n_chunks, int dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  g_err.clear();
  fakv_status s = check_decode(q, k, v, o, B, h_q, h_kv, d, S_kv, n_chunks, dtype);
  if (s != FAKV_OK) return s;
  const size_t need = splitkv_decode_workspace_bytes(B, h_q, d, n_chunks);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(FAKV_EINVAL, "workspace too small: need %zu bytes, got %zu", need, workspace_bytes);
  if (!aligned16(workspace)) return fail(FAKV_EINVAL, "workspace must be 16-byte aligned");
  return enqueue_decode(q, k, v, o, B, h_q, h_kv, d, S_kv, n_chunks, static_cast<char*>(workspace), stream);
}

fakv_status splitkv_decode_noalloc(const void* q, const void* k, const void* v, void* o, int B, int h_q,
                                   int h_kv, int d, int S_kv, int n_chunks, int dtype, void* stream) {
  g_err.clear();
  fakv_status s = check_decode(q, k, v, o, B, h_q, h_kv, d, S_kv, n_chunks, dtype);
  if (s != FAKV_OK) return s;
  const size_t need = splitkv_decode_workspace_bytes(B, h_q, d, n_chunks);
  if (need > (size_t)FAKV_DECODE_SCRATCH_BYTES)
    return fail(FAKV_EINVAL,
                "splitkv_decode_noalloc: partials of n_chunks * B * h_q * (d + 2) fp32 need %zu bytes, "
                "beyond the library's %zu-byte scratch; use splitkv_decode with a workspace",
                need, (size_t)FAKV_DECODE_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((s = scratch_of_current_device(&ws)) != FAKV_OK) return s;
  return enqueue_decode(q, k, v, o, B, h_q, h_kv, d, S_kv, n_chunks, static_cast<char*>(ws), stream);
}

fakv_status fakv_jagged_worklist(const int32_t* seq_offsets, int n_seqs, int total_tokens, int BQ,
                                 int32_t* items, int32_t* n_items, size_t capacity, void* stream) {
  g_err.clear();
  if (!seq_offsets || !items || !n_items) return fail(FAKV_EINVAL, "null pointer argument");
  if (n_seqs < 1 || total_tokens < 0 || BQ < 1)
    return fail(FAKV_EINVAL, "need n_seqs >= 1, total_tokens >= 0, BQ >= 1");
  const size_t cap = worklist_capacity(total_tokens, n_seqs, BQ);
  if (capacity < cap) return fail(FAKV_EINVAL, "capacity %zu below the bound %zu", capacity, cap);
  if (cap > 0x7fffffffull) return fail(FAKV_EINVAL, "worklist too large");
  hipError_t e = fakv::launch_worklist(seq_offsets, n_seqs, total_tokens, BQ, items, n_items,
                                       (int)cap, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail("worklist launch", e);
  return FAKV_OK;
}

}  // extern "C"
