// merge.hip -- n-way merge of (m, l, O) triplets and the final O / l.
//
// The merge rule is the online-softmax step of the prefill page's ring loop
// and of the decode page's fan-out: the merged max m' is the max of the parts,
// every part is rescaled by exp(m_c - m') and the l's and O's add.  Applied to
// all n parts of a row at once it reads: m' = max_c m_c, l' = sum_c l_c
// exp(m_c - m'), O' = sum_c O_c exp(m_c - m') -- the root of a one-level merge
// tree, equal in exact arithmetic to any pairwise order.  Sums run in part
// order c = 0 .. n-1, so results are reproducible bit for bit.  Parts with
// m = -inf (empty chunks) get weight 0.
//
// Threads: one per (row, 4 consecutive dims); a row's threads read its parts'
// m / l redundantly (cached) and their own 16-byte slice of each O part.
#include "fakv_device.h"
#include "fakv_kernels.h"

namespace fakv {

template <int D>
__global__ __launch_bounds__(256)
void lse_merge_kernel(MergeParams p) {
  constexpr int TPR = D / 4;               // threads per row
  constexpr int RPB = 256 / TPR;           // rows per block
  const int t = threadIdx.x % TPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= p.rows) return;
  const size_t rows = (size_t)p.rows;

  float M = neg_inf();
  for (int c = 0; c < p.n_parts; ++c) M = fmaxf(M, p.m_parts[(size_t)c * rows + row]);
  const float Mu = (M == neg_inf()) ? 0.f : M;

  float l = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < p.n_parts; ++c) {
    const size_t idx = (size_t)c * rows + row;
    const float wgt = fast_exp2((p.m_parts[idx] - Mu) * kLog2e);
    l += wgt * p.l_parts[idx];
    const f32x4 x = *reinterpret_cast<const f32x4*>(p.o_parts + idx * D + 4 * t);
    o += wgt * x;
  }
  const float inv = 1.f / l;
  if (p.out_bf16) {
    u32x2 x = {pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.o_out) + row * D + 4 * t) = x;
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.o_out) + row * D + 4 * t) = o * inv;
  }
  if (p.lse_out != nullptr && t == 0) p.lse_out[row] = M + logf(l);
}

template <int D>
static hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  constexpr int RPB = 256 / (D / 4);
  const long long grid = ((long long)p.rows + RPB - 1) / RPB;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(lse_merge_kernel<D>, dim3((unsigned)grid), dim3(256), 0, stream, p);
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
