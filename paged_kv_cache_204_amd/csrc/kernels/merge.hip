// Log-sum-exp merge of partial softmax states computed over disjoint key
// sets (key chunks and shared-prefix segments of one query):
//   M = max_i lse_i,  w_i = 2^(lse_i - M),  out = sum_i w_i o_i / sum_i w_i,
//   lse = (M + log2 sum_i w_i) * ln 2.
// Partial states hold normalised o_i and a base-2 lse_i (-inf for a key set
// the row could not see).  Grid: merged query vectors x chunks of 256
// (q head, 4 dims) units; each thread reads its float4 of every partial.
// Up to kMergeInline part rows travel inside the merge row itself, so all
// partial loads leave in one round trip.
#include <math.h>

#include "../kernels.hpp"
#include "common.hpp"

namespace pkv {
namespace {

__device__ __forceinline__ void merge_write(const MergeParams& p, const MergeRow& mr, int hq, int d,
                                            float mx, float wsum, float4 acc) {
  const float inv = 1.f / wsum;
  const size_t orow = static_cast<size_t>(mr.q_index) * p.Hq + hq;
  *reinterpret_cast<float4*>(p.out + orow * p.D + d) =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (p.lse && d == 0) p.lse[orow] = (mx + log2f(wsum)) * kLn2;
}

// merges leads the arguments so that it arrives preloaded in SGPRs
__global__ __launch_bounds__(256) void merge_kernel(const MergeRow* __restrict__ merges, MergeParams p) {
  const MergeRow mr = merges[blockIdx.x];
  const int per_head = p.D / 4;
  const int u = blockIdx.y * blockDim.x + threadIdx.x;
  if (u >= p.Hq * per_head) return;
  const int hq = u / per_head;
  const int d = (u % per_head) * 4;
  if (mr.n_parts <= kMergeInline) {
    // part rows come with the merge row: every partial is requested at once
    float l[kMergeInline];
    float4 v[kMergeInline];
#pragma unroll
    for (int k = 0; k < kMergeInline; ++k) {
      if (k < mr.n_parts) {
        const size_t row = static_cast<size_t>(mr.inl[k]) + hq;
        l[k] = p.part_lse[row];
        v[k] = *reinterpret_cast<const float4*>(p.part_o + row * p.D + d);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMergeInline; ++k)
      if (k < mr.n_parts) mx = fmaxf(mx, l[k]);
    float wsum = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < kMergeInline; ++k) {
      if (k < mr.n_parts) {
        const float w = (l[k] == -INFINITY) ? 0.f : exp2f(l[k] - mx);
        wsum += w;
        acc.x = fmaf(w, v[k].x, acc.x);
        acc.y = fmaf(w, v[k].y, acc.y);
        acc.z = fmaf(w, v[k].z, acc.z);
        acc.w = fmaf(w, v[k].w, acc.w);
      }
    }
    merge_write(p, mr, hq, d, mx, wsum, acc);
    return;
  }
  const int32_t* parts = p.parts + mr.parts_off;
  float mx = -INFINITY;
#pragma unroll 4
  for (int k = 0; k < mr.n_parts; ++k) mx = fmaxf(mx, p.part_lse[parts[k] + hq]);
  float wsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int k = 0; k < mr.n_parts; ++k) {
    const size_t row = static_cast<size_t>(parts[k]) + hq;
    const float l = p.part_lse[row];
    const float w = (l == -INFINITY) ? 0.f : exp2f(l - mx);
    const float4 v = *reinterpret_cast<const float4*>(p.part_o + row * p.D + d);
    wsum += w;
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
  merge_write(p, mr, hq, d, mx, wsum, acc);
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, int32_t n_rows, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  const int units = p.Hq * (p.D / 4);
  const dim3 grid(static_cast<uint32_t>(n_rows), static_cast<uint32_t>((units + 255) / 256));
  hipLaunchKernelGGL(merge_kernel, grid, dim3(256), 0, s, p.merges, p);
  return hipGetLastError();
}

}  // namespace pkv
