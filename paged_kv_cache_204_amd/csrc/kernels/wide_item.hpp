// Body of the dense-tile attention kernel (one work item for one kv head in
// the caller's LDS), shared by that kernel and the tree decode kernel; the
// method (score products, online softmax with bf16 P and its residual term,
// P V products, the load ring) is described beside the dense-tile kernel.
#pragma once

#include <math.h>

#include <type_traits>
#include <utility>

#include "../kernels.hpp"
#include "common.hpp"
#include "tile.hpp"

namespace pkv {
namespace dense {

constexpr float kLoShare = 16.f;   // residual term while a weight exceeds sum / 16

template <int D, int RING>
struct WideSmem {
  char k[RING][kStep * D * 2];
  char v[RING][kStep * D * 2];
};

// f(integral_constant<int, I>) for I in the sequence, in order
template <class F, int... I>
__device__ __forceinline__ void unrolled(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}

// One work item for kv head h, in the caller's LDS: W waves of NT tiles
// each (W * NT * 16 rows); tile t of the item is held by wave t % W.  RING
// K/V tiles in LDS: the loads run RING - 2 steps ahead of the step whose
// scores are formed.  NT is fixed at compile time so that a step's code has
// no per-tile branches: tiles past the item's rows compute on zero queries
// and are never stored.  Writes out / lse, or partial states when the item
// has partial rows.
template <int D, int W, int NT, int RING, int UNROLL>
__device__ __forceinline__ void wide_item(const int item, const int h, const WorkItem* __restrict__ items,
                                          const int32_t* __restrict__ blocks,
                                          const RowGroup* __restrict__ groups,
                                          const uint16_t* __restrict__ q, int32_t stride,
                                          const AttnParams& p, WideSmem<D, RING>& sm, int32_t* blk_s) {
  constexpr int NK = D / 32;
  constexpr int ND = D / 16;
  constexpr int CPR = D / 8;
  constexpr int RUNS = kStep * CPR / 64;    // 1 KB runs per tile
  constexpr int IPW = 2 * RUNS / W;         // K and V runs each wave loads per step
  static_assert(IPW * W == 2 * RUNS, "a step's runs split evenly over the waves");
  static_assert(RING >= 4 && RING % 2 == 0, "ring of an even number of tiles");
  static_assert(UNROLL == 2 || UNROLL == RING, "unrolled by two or by the ring");
  static_assert(IPW * (RING - 2) < 64, "load-counter range");
  const int tid = threadIdx.x;
  const int32_t* lst = blocks + static_cast<size_t>(item) * stride;
  for (int i = tid; i < stride; i += 64 * W) blk_s[i] = lst[i];
  const WorkItem it = items[item];
  lds_barrier();

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int G = p.G;
  const int R = it.n_grp * G;

  bf16x8 qf[NT][NK];
  uint64_t anc[NT];
  bool row_ok[NT];
  size_t dst_row[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int r = (wave + W * j) * 16 + l16;
    row_ok[j] = r < R;
    anc[j] = 0;
    dst_row[j] = 0;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) qf[j][kk] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
    if (row_ok[j]) {
      const RowOf ro = row_of(p, r);
      const RowGroup g = groups[it.grp_off + ro.grp];
      const int hq = h * G + ro.head;
      const uint16_t* qrow = q + (static_cast<size_t>(g.q_index) * p.Hq + hq) * D;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        qf[j][kk] = *reinterpret_cast<const bf16x8*>(qrow + 32 * kk + 8 * g4);
      anc[j] = (static_cast<uint64_t>(g.anc_hi) << 32) | g.anc_lo;
      dst_row[j] = it.part_base < 0
                       ? static_cast<size_t>(g.q_index) * p.Hq + hq
                       : static_cast<size_t>(it.part_base) + static_cast<size_t>(ro.grp) * p.Hq + hq;
    }
  }

  // o[j][ND] is the row sum of P: the P V product against a tile of ones
  // (all four entries of a lane hold the sum of its row), so the softmax
  // denominator comes from the same rounded weights as the numerator and
  // costs one MFMA instead of a chain of adds and cross-lane sums
  float m_run[NT];
  f32x4 o[NT][ND + 1];
  f32x4 s0[NT][2], s1[NT][2];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    m_run[j] = -INFINITY;
#pragma unroll
    for (int dt = 0; dt <= ND; ++dt) o[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const uint4* kb = layer_head_base(p, p.k_pool, h, D);
  const uint4* vb = layer_head_base(p, p.v_pool, h, D);
  const uint32_t blk_chunks = static_cast<uint32_t>(p.Hkv * p.B * D / 8);
  const int t_last = it.n_tok - 1;
  const int nsteps = (it.n_tok + kStep - 1) / kStep;
  // steps before this one are full (every key visible to every row)
  const int nfull = min(it.n_tok, it.tail_start) / kStep;
  // Run u of a step (K runs first, then V): lane i fills chunk slot
  // c = 64 (u % RUNS) + i of its tile, i.e. row c / CPR and chunk
  // (c % CPR) ^ tile_swz(row).  Tokens past the end re-read the last token
  // (masked in the softmax), so every run stays inside the pool.
  auto issue = [&](int s) __attribute__((always_inline)) {
    const int t0 = s * kStep;
    const int b = s % RING;
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      const int j = wave * IPW + u;
      const int c = (j % RUNS) * 64 + lane;
      const int r = c / CPR;
      const int ch = (c % CPR) ^ tile_swz<D>(r);
      const int t = min(t0 + r, t_last);
      const uint32_t ci = chunk_index(blk_s[t >> p.log2B], blk_chunks, (t & (p.B - 1)) * CPR + ch);
      char* dst = (j >= RUNS ? sm.v[b] : sm.k[b]) + (j % RUNS) * 1024;
      lds_dma16((j >= RUNS ? vb : kb) + ci, dst);
    }
  };
  // this wave's runs of a step have landed once at most `later` younger
  // steps (IPW runs each) are still in flight
  auto landed = [&](int later) __attribute__((always_inline)) { wait_vmcnt_steps<IPW, RING - 2>(later); };

  // S^T of step s for this wave's tiles
  auto scores = [&](int s, f32x4 (&acc)[NT][2], int b) __attribute__((always_inline)) {
    const char* kt = sm.k[b];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      acc[j][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + tile_byte<D>(16 * tt + l16, 4 * kk + g4));
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[j][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[j][kk], acc[j][tt], 0, 0, 0);
      }
    }
  };

  // Softmax of a step, first half: mask (MASK: some key of the step is past
  // the item's end or in the draft-tree tail), row max, and the weights.  A
  // row's reference max m moves only when the row's max passes it by more
  // than kSlack -- to that max -- so P <= 2^kSlack and the O rescale (the
  // rare branch afterwards, which leaves the weights alone) is rare after the
  // first steps.  The weights thus stay in one block with the score products
  // issued just before, which they interleave with.
  float sv[NT][8], pv[NT][8], mx[NT], m_new[NT];
  auto soft_a = [&](auto mask_tag, int s, f32x4 (&acc)[NT][2]) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int t0 = s * kStep;
    bool grow = false;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[j][4 * tt + i] = acc[j][tt][i];
      if constexpr (MASK) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tok = t0 + 16 * (e >> 2) + 4 * g4 + (e & 3);
          bool vis = tok < it.n_tok;
          if (vis && tok >= it.tail_start) vis = (anc[j] >> (it.tail_node0 + tok - it.tail_start)) & 1ull;
          if (!vis) sv[j][e] = -INFINITY;
        }
      }
      float m = sv[j][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) m = fmaxf(m, sv[j][e]);
      mx[j] = xor32_max(xor16_max(m)) * p.scale_log2;
      m_new[j] = mx[j] > m_run[j] + kSlack ? mx[j] : m_run[j];
      grow = grow || m_new[j] != m_run[j];
      const float m_use = (m_new[j] == -INFINITY) ? 0.f : m_new[j];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[j][e] = fast_exp2(fmaf(sv[j][e], p.scale_log2, -m_use));
      // the weights are taken here, before the rescale branch (the compiler
      // would otherwise sink them past it, away from the score products)
      asm volatile("" ::"v"(pv[j][0]), "v"(pv[j][1]), "v"(pv[j][2]), "v"(pv[j][3]), "v"(pv[j][4]),
                   "v"(pv[j][5]), "v"(pv[j][6]), "v"(pv[j][7]));
    }
    return __ballot(grow) != 0;
  };
  auto regrow = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const float alpha = (m_run[j] == -INFINITY) ? 0.f : fast_exp2(m_run[j] - m_new[j]);
#pragma unroll
      for (int dt = 0; dt <= ND; ++dt) o[j][dt] *= alpha;
      m_run[j] = m_new[j];
    }
  };
  // Second half: the sums, bf16 P, and O^T += V^T P^T; the residual term
  // follows when some row still has a weight above its running sum / 64.
  auto soft_b = [&](int s, int b) __attribute__((always_inline)) {
    bf16x8 pf[NT];
    bool need_lo = false;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      uint32_t ph[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) ph[e >> 1] = pack_bf16x2(pv[j][e], pv[j][e + 1]);
      uint4 hv = make_uint4(ph[0], ph[1], ph[2], ph[3]);
      pf[j] = *reinterpret_cast<bf16x8*>(&hv);
      // the row's largest weight of this step against its sum over the
      // steps before (that step's ones product has long completed)
      const float m_use = (m_run[j] == -INFINITY) ? 0.f : m_run[j];
      const float p_top = mx[j] == -INFINITY ? 0.f : fast_exp2(mx[j] - m_use);
      need_lo = need_lo || (row_ok[j] && p_top * kLoShare > o[j][ND][0]);
    }
    // lane (l16, g4) of a 16-lane group names 4 dims of one token row; the
    // transposed read hands lane i of the group dim 16 dt + i of 4 tokens
    const char* vt = sm.v[b];
    auto vop = [&](int dt) __attribute__((always_inline)) {
      const int r = 4 * g4 + (l16 >> 2);
      const int c = 2 * dt + ((l16 & 3) >> 1);
      const int off = (l16 & 1) * 8;
      const v4i16 vlo = lds_read_tr16(vt + tile_byte<D>(r, c) + off);
      const v4i16 vhi = lds_read_tr16(vt + tile_byte<D>(16 + r, c) + off);
      return bf16x8{vlo[0], vlo[1], vlo[2], vlo[3], vhi[0], vhi[1], vhi[2], vhi[3]};
    };
    const bf16x8 ones = {0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80};
#pragma unroll
    for (int dt = 0; dt <= ND; ++dt) {
      const bf16x8 a = dt < ND ? vop(dt) : ones;
#pragma unroll
      for (int j = 0; j < NT; ++j)
        o[j][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[j], o[j][dt], 0, 0, 0);
    }
    if (__ballot(need_lo)) {
      // residual P - bf16(P) as a second term for this step
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const uint4 hv = *reinterpret_cast<const uint4*>(&pf[j]);
        const uint32_t ph[4] = {hv.x, hv.y, hv.z, hv.w};
        uint32_t pl[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2)
          pl[e >> 1] = pack_bf16x2(pv[j][e] - __uint_as_float(ph[e >> 1] << 16),
                                   pv[j][e + 1] - __uint_as_float(ph[e >> 1] & 0xFFFF0000u));
        uint4 lv = make_uint4(pl[0], pl[1], pl[2], pl[3]);
        const bf16x8 pfl = *reinterpret_cast<bf16x8*>(&lv);
#pragma unroll
        for (int dt = 0; dt <= ND; ++dt)
          o[j][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dt < ND ? vop(dt) : ones, pfl, o[j][dt], 0, 0, 0);
      }
    }
  };

#pragma unroll
  for (int u = 0; u < RING - 1; ++u)
    if (u < nsteps) issue(u);
  // The query operands and masks were loaded first; taking them here makes
  // the compiler's wait for them land before the loop, not inside it.
#pragma unroll
  for (int j = 0; j < NT; ++j) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) asm volatile("" : "+v"(qf[j][kk]));
    asm volatile("" : "+v"(anc[j]));
  }
  landed(min(nsteps - 1, RING - 2));
  lds_barrier();
  scores(0, s0, 0);
  // step s (not the last): make step s + 1's tile visible, refill the slot
  // step s - 1 used (every wave read it before the barrier), then S(s + 1)
  // together with the first softmax half of step s, and its second half.
  // The steps before nfull run in one loop and the masked ones in another,
  // so that no branch separates a step's score products from its weights.
  // slot: s % RING, a constant where the caller knows it (else -1)
  auto step = [&](auto mask_tag, int s, f32x4 (&cur)[NT][2], f32x4 (&nxt)[NT][2],
                  auto slot) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot)::value;
    const int b = SL >= 0 ? SL : s % RING;
    landed(min(nsteps - 2 - s, RING - 3));
    lds_barrier();
    if (s + RING - 1 < nsteps) issue(s + RING - 1);
    scores(s + 1, nxt, (b + 1) % RING);
    const bool grow = soft_a(mask_tag, s, cur);
    if (grow) regrow();
    soft_b(s, b);
  };
  auto shift = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      s0[j][0] = s1[j][0];
      s0[j][1] = s1[j][1];
    }
  };
  int s = 0;
  const int lim = min(nfull, nsteps - 1);   // unmasked steps that have a next step
  // UNROLL steps per turn (UNROLL = RING: the slots are constants, so the
  // LDS reads take them as immediate offsets; 2: fewer registers)
  for (; s + UNROLL - 1 < lim; s += UNROLL) {
    unrolled(std::make_integer_sequence<int, UNROLL>{}, [&](auto c) __attribute__((always_inline)) {
      constexpr int C = decltype(c)::value;
      constexpr int SL = UNROLL == RING ? C : -1;
      if constexpr (C % 2 == 0)
        step(std::false_type{}, s + C, s0, s1, std::integral_constant<int, SL>{});
      else
        step(std::false_type{}, s + C, s1, s0, std::integral_constant<int, SL>{});
    });
  }
  for (; s + 1 < lim; s += 2) {
    step(std::false_type{}, s, s0, s1, std::integral_constant<int, -1>{});
    step(std::false_type{}, s + 1, s1, s0, std::integral_constant<int, -1>{});
  }
  if (s < lim) {
    step(std::false_type{}, s, s0, s1, std::integral_constant<int, -1>{});
    shift();
    ++s;
  }
  for (; s + 1 < nsteps; ++s) {
    step(std::true_type{}, s, s0, s1, std::integral_constant<int, -1>{});
    shift();
  }
  {
    const bool grow = s < nfull ? soft_a(std::false_type{}, s, s0) : soft_a(std::true_type{}, s, s0);
    if (grow) regrow();
    soft_b(s, s % RING);
  }
  // every run has landed (the last step's wait covered the last issue)
  wait_vmcnt<0>();

#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const float l = o[j][ND][0];
    if (!row_ok[j]) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* dst = (it.part_base < 0 ? p.out : p.part_o) + dst_row[j] * D;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      const f32x4 v = o[j][dt] * inv;
      *reinterpret_cast<float4*>(dst + 16 * dt + 4 * g4) = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (g4 == 0) {
      if (it.part_base < 0) {
        if (p.lse) p.lse[dst_row[j]] = (m_run[j] + log2f(l)) * kLn2;
      } else {
        p.part_lse[dst_row[j]] = l > 0.f ? m_run[j] + log2f(l) : -INFINITY;
      }
    }
  }
}

}  // namespace dense
}  // namespace pkv
