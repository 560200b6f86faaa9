// Paged attention on the matrix cores, for work items whose query tile is a
// real dense contraction: draft-tree verify (every node x the GQA heads of a
// kv head, CAST page, technical summary "Problem": the target checks the
// whole draft tree in one pass) and shared-prefix segments read by many
// queries at once.
//
// Workgroup: 8 waves; wave w owns RT row tiles of 16 rows (RT = 1 or 2), so an
// item holds up to 128 * RT rows.  Keys stream through LDS 32 tokens at a
// time (two 16-token MFMA tiles), double buffered, each token's address taken
// from the block table (staged in LDS once per item):
//   S^T = K Q^T  with v_mfma_f32_16x16x32_bf16 (A = K rows from LDS,
//                B = Q rows held in registers).  The accumulator layout gives
//                each lane 4 tokens of ONE query row, so the softmax max/sum
//                need only two cross-lane steps (lanes l, l^16, l^32, l^48).
//   P        = exp2(S * scale * log2 e - m), rounded to bf16; with the lane's
//                8 tokens it is exactly the B operand of the next product.
//   O^T     += V^T P^T (A = V^T from LDS, stored transposed while staging).
//                O^T keeps each lane on the same query row again, so the
//                online-softmax rescale of O is lane local.
// Draft-tree tail tokens are masked per row by the node's ancestor-or-self
// bits.  Output: final out / lse, or normalised partial states for the merge.
#include <math.h>

#include "../kernels.hpp"
#include "common.hpp"

namespace pkv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kStep = 32;      // key tokens per step
constexpr int kMaxBlk = 512;   // block ids of one item staged in LDS

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int D, int RT>
__global__ __launch_bounds__(kThreads) void attn_mfma_kernel(AttnParams p) {
  constexpr int KP = D + 8;        // K tile row pitch (bf16 elements)
  constexpr int VP = kStep + 4;    // V^T row pitch (bf16 elements), 72 bytes
  constexpr int NK = D / 32;       // MFMA steps over head_dim for S
  constexpr int ND = D / 16;       // 16-wide head_dim tiles of O
  constexpr int CPR = D / 8;       // 16-byte chunks per K/V row
  __shared__ __align__(16) uint16_t k_s[2][kStep][KP];
  __shared__ __align__(16) uint16_t vt_s[2][D][VP];
  __shared__ int32_t blk_s[kMaxBlk];

  const WorkItem it = p.items[blockIdx.x];
  const int h = blockIdx.y;
  const int G = p.G;
  const int R = it.n_grp * G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  const int nblk = (it.n_tok + p.B - 1) >> p.log2B;
  for (int i = tid; i < nblk; i += kThreads) blk_s[i] = p.blocks[it.blk_off + i];

  // this lane's query row in each of its row tiles
  bf16x8 qf[RT][NK];
  uint64_t anc[RT];
  bool row_ok[RT];
  size_t dst_row[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = (wave * RT + rt) * 16 + l16;
    row_ok[rt] = r < R;
    anc[rt] = 0;
    dst_row[rt] = 0;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) qf[rt][kk] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
    if (row_ok[rt]) {
      const RowGroup g = p.groups[it.grp_off + r / G];
      const int hq = h * G + r % G;
      const uint16_t* qrow = p.q + (static_cast<size_t>(g.q_index) * p.Hq + hq) * D;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        qf[rt][kk] = *reinterpret_cast<const bf16x8*>(qrow + 32 * kk + 8 * g4);
      anc[rt] = (static_cast<uint64_t>(g.anc_hi) << 32) | g.anc_lo;
      dst_row[rt] = it.part_base < 0
                        ? static_cast<size_t>(g.q_index) * p.Hq + hq
                        : static_cast<size_t>(it.part_base) + static_cast<size_t>(r / G) * p.Hq + hq;
    }
  }
  const int rows_here = R - wave * RT * 16;   // rows of this wave (may be <= 0)
  const bool active = rows_here > 0;

  float m_run[RT], l_run[RT];
  f32x4 o[RT][ND];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // staging: thread -> (token, 16-byte chunk) of the K and V tiles
  const int ld_tok = tid / CPR;
  const int ld_c = tid % CPR;
  const bool ld_on = tid < kStep * CPR;
  const size_t blk_stride = static_cast<size_t>(p.Hkv) * p.B * D;
  const size_t base = static_cast<size_t>(p.layer) * p.N * blk_stride + static_cast<size_t>(h) * p.B * D;
  const uint16_t* kb = p.k_pool + base;
  const uint16_t* vb = p.v_pool + base;

  __syncthreads();  // blk_s

  uint4 kr = make_uint4(0, 0, 0, 0), vr = make_uint4(0, 0, 0, 0);
  auto fetch = [&](int t0) {
    const int t = t0 + ld_tok;
    if (ld_on && t < it.n_tok) {
      const int blk = blk_s[t >> p.log2B];
      const size_t off = static_cast<size_t>(blk) * blk_stride + static_cast<size_t>(t & (p.B - 1)) * D + ld_c * 8;
      kr = *reinterpret_cast<const uint4*>(kb + off);
      vr = *reinterpret_cast<const uint4*>(vb + off);
    } else {
      kr = make_uint4(0, 0, 0, 0);   // zero K/V past the end: masked, and 0 * V stays finite
      vr = make_uint4(0, 0, 0, 0);
    }
  };

  const int nsteps = (it.n_tok + kStep - 1) / kStep;
  fetch(0);
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (ld_on) {
      *reinterpret_cast<uint4*>(&k_s[buf][ld_tok][ld_c * 8]) = kr;
      const uint32_t w[4] = {vr.x, vr.y, vr.z, vr.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vt_s[buf][ld_c * 8 + 2 * j][ld_tok] = static_cast<uint16_t>(w[j] & 0xFFFFu);
        vt_s[buf][ld_c * 8 + 2 * j + 1][ld_tok] = static_cast<uint16_t>(w[j] >> 16);
      }
    }
    __syncthreads();
    if (s + 1 < nsteps) fetch((s + 1) * kStep);
    if (!active) continue;

    const int t0 = s * kStep;
    // ---- S^T = K Q^T --------------------------------------------------------
    f32x4 sacc[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      sacc[rt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      sacc[rt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&k_s[buf][16 * tt + l16][32 * kk + 8 * g4]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          sacc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[rt][kk], sacc[rt][tt], 0, 0, 0);
      }
    }
    // ---- online softmax, lane-local per row ----------------------------------
    const bool full = t0 + kStep <= it.n_tok && t0 + kStep <= it.tail_start;
    bf16x8 pf[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float sv[8];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[4 * tt + i] = sacc[rt][tt][i] * p.scale_log2;
      if (!full) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int tok = t0 + 16 * (j >> 2) + 4 * g4 + (j & 3);
          bool vis = tok < it.n_tok;
          if (vis && tok >= it.tail_start)
            vis = (anc[rt] >> (it.tail_node0 + tok - it.tail_start)) & 1ull;
          if (!vis) sv[j] = -INFINITY;
        }
      }
      float mx = sv[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sv[j]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[rt], mx);
      const float alpha = (m_run[rt] == -INFINITY) ? 0.f : exp2f(m_run[rt] - m_new);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      float ps = 0.f;
      uint32_t pk[4];
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float p0 = exp2f(sv[j] - m_use);
        const float p1 = exp2f(sv[j + 1] - m_use);
        ps += p0 + p1;
        pk[j >> 1] = bf16_rne_bits(p0) | (bf16_rne_bits(p1) << 16);
      }
      l_run[rt] = l_run[rt] * alpha + ps;
      m_run[rt] = m_new;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) o[rt][dt] *= alpha;
      uint4 pv = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      pf[rt] = *reinterpret_cast<bf16x8*>(&pv);
    }
    // ---- O^T += V^T P^T -----------------------------------------------------
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      const uint2 lo = *reinterpret_cast<const uint2*>(&vt_s[buf][16 * dt + l16][4 * g4]);
      const uint2 hi = *reinterpret_cast<const uint2*>(&vt_s[buf][16 * dt + l16][16 + 4 * g4]);
      uint4 av = make_uint4(lo.x, lo.y, hi.x, hi.y);
      const bf16x8 a = *reinterpret_cast<bf16x8*>(&av);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[rt], o[rt][dt], 0, 0, 0);
    }
  }

  if (!active) return;
  // ---- epilogue: full row sums, normalise, write --------------------------
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float l = l_run[rt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (!row_ok[rt]) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* dst = (it.part_base < 0 ? p.out : p.part_o) + dst_row[rt] * D;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      const f32x4 v = o[rt][dt] * inv;
      *reinterpret_cast<float4*>(dst + 16 * dt + 4 * g4) = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (g4 == 0) {
      if (it.part_base < 0) {
        if (p.lse) p.lse[dst_row[rt]] = (m_run[rt] + log2f(l)) * kLn2;
      } else {
        p.part_lse[dst_row[rt]] = l > 0.f ? m_run[rt] + log2f(l) : -INFINITY;
      }
    }
  }
}

}  // namespace

hipError_t launch_attn_mfma(const AttnParams& p, int32_t n_items, int32_t head_dim,
                            int32_t row_tiles, hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(n_items), static_cast<uint32_t>(p.Hkv));
  const dim3 block(kThreads);
  if (head_dim == 64 && row_tiles == 1)
    hipLaunchKernelGGL((attn_mfma_kernel<64, 1>), grid, block, 0, s, p);
  else if (head_dim == 64 && row_tiles == 2)
    hipLaunchKernelGGL((attn_mfma_kernel<64, 2>), grid, block, 0, s, p);
  else if (head_dim == 128 && row_tiles == 1)
    hipLaunchKernelGGL((attn_mfma_kernel<128, 1>), grid, block, 0, s, p);
  else if (head_dim == 128 && row_tiles == 2)
    hipLaunchKernelGGL((attn_mfma_kernel<128, 2>), grid, block, 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
