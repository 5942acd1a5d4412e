// merge.hip -- n-way merge of (m, l, O) triplets and the final O / l.
//
// The merge rule is the online-softmax step of the prefill page's ring loop
// and of the decode page's fan-out: the merged max m' is the max of the parts,
// every part is rescaled by exp(m_c - m') and the l's and O's add.  Applied to
// all n parts of a row at once it reads: m' = max_c m_c, l' = sum_c l_c
// exp(m_c - m'), O' = sum_c O_c exp(m_c - m') -- the root of a one-level merge
// tree, equal in exact arithmetic to any pairwise order.  Parts with
// m = -inf (empty chunks) get weight 0.  A row whose parts are all empty
// merges to the identity (-inf, 0, 0): its output row is written as zeros and
// its lse as -inf (ln of an empty sum), never 0/0.
//
// One workgroup per row: thread t owns 4 consecutive dims (t mod D/4) of the
// parts c = g, g + G, g + 2G, ... of part group g = t / (D/4), G = 1024/D.
// The common max comes from an LDS max over the groups; each group sums its
// parts in order, then the G group sums are added in group order -- a fixed
// order, so results are reproducible bit for bit.
#include <type_traits>
#include <utility>

#include "fakv_device.h"
#include "fakv_kernels.h"

namespace fakv {

template <int D>
__global__ __launch_bounds__(256)
void lse_merge_kernel(MergeParams p) {
  constexpr int TPR = D / 4;               // threads per part group
  constexpr int G = 256 / TPR;             // part groups
  __shared__ float s_m[G];
  __shared__ f32x4 s_o[G][TPR];
  __shared__ float s_l[G];
  const int t = threadIdx.x % TPR;
  const int grp = threadIdx.x / TPR;
  const size_t row = blockIdx.x;
  const size_t rows = (size_t)p.rows;

  // Both loops unrolled so that the loads of several parts are in flight at
  // once (each part's values are independent; only the sums are ordered).
  float M = neg_inf();
#pragma unroll 8
  for (int c = grp; c < p.n_parts; c += G) M = fmaxf(M, p.m_parts[(size_t)c * rows + row]);
  if (t == 0) s_m[grp] = M;
  __syncthreads();
  M = s_m[0];
#pragma unroll
  for (int q = 1; q < G; ++q) M = fmaxf(M, s_m[q]);
  const float Mu = (M == neg_inf()) ? 0.f : M;

  // Parts in batches of U: the batch's loads first (indices clamped to the
  // last part, so every address is valid), then the in-order sums of the
  // parts that exist.
  constexpr int U = 4;
  float l = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  if (p.n_parts <= G) {                    // at most one part per group
    if (grp < p.n_parts) {
      const size_t idx = (size_t)grp * rows + row;
      const float wgt = fast_exp2((p.m_parts[idx] - Mu) * kLog2e);
      l = wgt * p.l_parts[idx];
      o = wgt * *reinterpret_cast<const f32x4*>(p.o_parts + idx * D + 4 * t);
    }
  } else {
    for (int c0 = grp; c0 < p.n_parts; c0 += U * G) {
      float mv[U], lv[U];
      f32x4 ov[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t idx = (size_t)min(c0 + u * G, p.n_parts - 1) * rows + row;
        mv[u] = p.m_parts[idx];
        lv[u] = p.l_parts[idx];
        ov[u] = *reinterpret_cast<const f32x4*>(p.o_parts + idx * D + 4 * t);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (c0 + u * G < p.n_parts) {
          const float wgt = fast_exp2((mv[u] - Mu) * kLog2e);
          l += wgt * lv[u];
          o += wgt * ov[u];
        }
      }
    }
  }
  s_o[grp][t] = o;
  if (t == 0) s_l[grp] = l;
  __syncthreads();
  if (grp != 0) return;
  l = s_l[0];
  o = s_o[0][t];
#pragma unroll
  for (int q = 1; q < G; ++q) {
    l += s_l[q];
    o += s_o[q][t];
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;   // all parts empty: O' = 0, written as 0
  if (p.out_bf16) {
    u32x2 x = {pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.o_out) + row * D + 4 * t) = x;
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.o_out) + row * D + 4 * t) = o * inv;
  }
  if (p.lse_out != nullptr && t == 0) p.lse_out[row] = l > 0.f ? M + logf(l) : neg_inf();
}

template <int D>
static hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(lse_merge_kernel<D>, dim3((unsigned)p.rows), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_lse_merge(const MergeParams& p, int d, hipStream_t stream) {
  switch (d) {
    case 64: return launch_merge<64>(p, stream);
    case 128: return launch_merge<128>(p, stream);
    case 256: return launch_merge<256>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fakv
