// Paged attention on the vector ALUs: one workgroup per (work item, kv head).
//
// A work item holds up to 16 query rows (row groups x the G query heads that
// share this kv head) and a run of key tokens reached through the block
// table.  Decode is bound by memory bandwidth (SGLang RadixAttention page,
// section on the KV-cache lifecycle), so the kernel is built around the K/V
// stream:
//   - each 64-token tile of K and V is loaded with coalesced 128-bit loads,
//     16 bytes per lane, every token's address taken from the block table,
//     and staged in LDS where all rows of the item reuse it -- the GQA head
//     group and every query that shares the blocks read each tile once;
//   - scores S = scale * Q K^T (fp32 accumulate on exact bf16 widening),
//     optional draft-tree mask on tail tokens;
//   - online softmax per row with 64-lane butterfly max / sum reductions
//     (exp2 domain), O = O * alpha + P V;
//   - epilogue writes final out / lse, or a normalised partial state for the
//     log-sum-exp merge when the item covers only part of a row's keys.
#include <math.h>

#include "../kernels.hpp"
#include "common.hpp"

namespace pkv {
namespace {

constexpr int kTile = 64;     // key tokens per tile (one per lane in the softmax)
constexpr int kMaxRows = 16;  // query rows per item
constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void attn_valu_kernel(AttnParams p) {
  constexpr int kPad = 8;          // bf16 row padding of the K tile
  constexpr int kCpr = D / 8;      // 16-byte chunks per head_dim row
  constexpr int kDpt = D / 16;     // output dims per thread (16 threads per row)
  __shared__ __align__(16) uint16_t k_s[kTile][D + kPad];
  __shared__ __align__(16) uint16_t v_s[kTile][D];
  __shared__ __align__(16) float q_s[kMaxRows][D];
  __shared__ float p_s[kMaxRows][kTile];
  __shared__ float m_s[kMaxRows], l_s[kMaxRows], a_s[kMaxRows];
  __shared__ uint64_t anc_s[kMaxRows];

  const WorkItem it = p.items[blockIdx.x];
  const int h = blockIdx.y;
  const int G = p.G;
  const int R = it.n_grp * G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  for (int e = tid; e < R * D; e += kThreads) {
    const int r = e / D, d = e % D;
    const RowGroup g = p.groups[it.grp_off + r / G];
    const size_t qoff = (static_cast<size_t>(g.q_index) * p.Hq + h * G + r % G) * D + d;
    q_s[r][d] = bf16_to_f32(p.q[qoff]);
  }
  if (tid < it.n_grp) {
    const RowGroup g = p.groups[it.grp_off + tid];
    anc_s[tid] = (static_cast<uint64_t>(g.anc_hi) << 32) | g.anc_lo;
  }
  if (tid < kMaxRows) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }

  const int ro = tid >> 4;               // output row of this thread
  const int d0 = (tid & 15) * kDpt;      // first output dim of this thread
  float o[kDpt];
#pragma unroll
  for (int k = 0; k < kDpt; ++k) o[k] = 0.f;

  const size_t blk_stride = static_cast<size_t>(p.Hkv) * p.B * D;
  const size_t base = static_cast<size_t>(p.layer) * p.N * blk_stride + static_cast<size_t>(h) * p.B * D;
  const uint16_t* kbase = p.k_pool + base;
  const uint16_t* vbase = p.v_pool + base;

  for (int t0 = 0; t0 < it.n_tok; t0 += kTile) {
    const int nt = min(kTile, it.n_tok - t0);
    __syncthreads();  // the previous tile's readers are done
    for (int c = tid; c < kTile * kCpr; c += kThreads) {
      const int tok = c / kCpr, col = (c % kCpr) * 8;
      if (tok < nt) {
        const int t = t0 + tok;
        const int blk = p.blocks[it.blk_off + (t >> p.log2B)];
        const size_t off = static_cast<size_t>(blk) * blk_stride + static_cast<size_t>(t & (p.B - 1)) * D + col;
        *reinterpret_cast<uint4*>(&k_s[tok][col]) = *reinterpret_cast<const uint4*>(kbase + off);
        *reinterpret_cast<uint4*>(&v_s[tok][col]) = *reinterpret_cast<const uint4*>(vbase + off);
      }
    }
    __syncthreads();
    for (int e = tid; e < R * kTile; e += kThreads) {
      const int r = e / kTile, t = e % kTile;
      float s = -INFINITY;
      const int tt = t0 + t;
      bool vis = t < nt;
      if (vis && tt >= it.tail_start) {
        const int node = it.tail_node0 + (tt - it.tail_start);
        vis = (anc_s[r / G] >> node) & 1ull;
      }
      if (vis) {
        float acc = 0.f;
#pragma unroll
        for (int d = 0; d < D; d += 8) {
          const uint4 w = *reinterpret_cast<const uint4*>(&k_s[t][d]);
          const float4 qa = *reinterpret_cast<const float4*>(&q_s[r][d]);
          const float4 qb = *reinterpret_cast<const float4*>(&q_s[r][d + 4]);
          acc = fmaf(qa.x, bf16_lo(w.x), acc);
          acc = fmaf(qa.y, bf16_hi(w.x), acc);
          acc = fmaf(qa.z, bf16_lo(w.y), acc);
          acc = fmaf(qa.w, bf16_hi(w.y), acc);
          acc = fmaf(qb.x, bf16_lo(w.z), acc);
          acc = fmaf(qb.y, bf16_hi(w.z), acc);
          acc = fmaf(qb.z, bf16_lo(w.w), acc);
          acc = fmaf(qb.w, bf16_hi(w.w), acc);
        }
        s = acc * p.scale_log2;
      }
      p_s[r][t] = s;
    }
    __syncthreads();
    for (int r = wave; r < R; r += kThreads / 64) {
      const float s = p_s[r][lane];
      const float m_old = m_s[r];
      const float m_new = fmaxf(m_old, wave_max(s));
      const float pr = (s == -INFINITY) ? 0.f : exp2f(s - m_new);
      const float lt = wave_sum(pr);
      const float alpha = (m_old == -INFINITY) ? 0.f : exp2f(m_old - m_new);
      p_s[r][lane] = pr;
      if (lane == 0) {
        l_s[r] = l_s[r] * alpha + lt;
        m_s[r] = m_new;
        a_s[r] = alpha;
      }
    }
    __syncthreads();
    if (ro < R) {
      const float alpha = a_s[ro];
#pragma unroll
      for (int k = 0; k < kDpt; ++k) o[k] *= alpha;
      for (int t = 0; t < nt; ++t) {
        const float pr = p_s[ro][t];
#pragma unroll
        for (int k = 0; k < kDpt; k += 2) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(&v_s[t][d0 + k]);
          o[k] = fmaf(pr, bf16_lo(w), o[k]);
          o[k + 1] = fmaf(pr, bf16_hi(w), o[k + 1]);
        }
      }
    }
  }
  __syncthreads();
  if (ro < R) {
    const float l = l_s[ro];
    const float m = m_s[ro];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const RowGroup g = p.groups[it.grp_off + ro / G];
    const int hq = h * G + ro % G;
    if (it.part_base < 0) {
      float* dst = p.out + (static_cast<size_t>(g.q_index) * p.Hq + hq) * D + d0;
#pragma unroll
      for (int k = 0; k < kDpt; ++k) dst[k] = o[k] * inv;
      if (p.lse && (tid & 15) == 0)
        p.lse[static_cast<size_t>(g.q_index) * p.Hq + hq] = (m + log2f(l)) * kLn2;
    } else {
      const size_t row = static_cast<size_t>(it.part_base) + static_cast<size_t>(ro / G) * p.Hq + hq;
      float* dst = p.part_o + row * D + d0;
#pragma unroll
      for (int k = 0; k < kDpt; ++k) dst[k] = o[k] * inv;
      if ((tid & 15) == 0) p.part_lse[row] = l > 0.f ? m + log2f(l) : -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_attn_valu(const AttnParams& p, int32_t n_items, int32_t head_dim, hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(n_items), static_cast<uint32_t>(p.Hkv));
  if (head_dim == 64)
    hipLaunchKernelGGL(attn_valu_kernel<64>, grid, dim3(kThreads), 0, s, p);
  else if (head_dim == 128)
    hipLaunchKernelGGL(attn_valu_kernel<128>, grid, dim3(kThreads), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
