// Log-sum-exp merge of partial softmax states computed over disjoint key
// sets (key chunks and shared-prefix segments of one query):
//   M = max_i lse_i,  w_i = 2^(lse_i - M),  out = sum_i w_i o_i / sum_i w_i,
//   lse = (M + log2 sum_i w_i) * ln 2.
// Partial states hold normalised o_i and a base-2 lse_i (-inf for a key set
// the row could not see).  One workgroup per merged query vector; threads
// walk (q head, dim) so the o_i reads are coalesced along head_dim.
#include <math.h>

#include "../kernels.hpp"
#include "common.hpp"

namespace pkv {
namespace {

__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  const MergeRow mr = p.merges[blockIdx.x];
  const int total = p.Hq * p.D;
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    const int hq = e / p.D, d = e % p.D;
    float mx = -INFINITY;
    for (int k = 0; k < mr.n_parts; ++k)
      mx = fmaxf(mx, p.part_lse[p.parts[mr.parts_off + k] + hq]);
    float wsum = 0.f, acc = 0.f;
    for (int k = 0; k < mr.n_parts; ++k) {
      const size_t row = static_cast<size_t>(p.parts[mr.parts_off + k]) + hq;
      const float l = p.part_lse[row];
      const float w = (l == -INFINITY) ? 0.f : exp2f(l - mx);
      wsum += w;
      acc = fmaf(w, p.part_o[row * p.D + d], acc);
    }
    p.out[(static_cast<size_t>(mr.q_index) * p.Hq + hq) * p.D + d] = acc / wsum;
    if (p.lse && d == 0)
      p.lse[static_cast<size_t>(mr.q_index) * p.Hq + hq] = (mx + log2f(wsum)) * kLn2;
  }
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, int32_t n_rows, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(static_cast<uint32_t>(n_rows)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace pkv
