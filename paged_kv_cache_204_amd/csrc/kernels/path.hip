// Path items of a tree decode plan: the narrow part of a decode call over
// prefix-sharing branches -- the levels of a search tree below its shared
// root, each leaf's own keys (SGLang RadixAttention page, measured benchmark:
// many branches over one parent; decode is bound by memory bandwidth,
// KV-cache lifecycle section).
//
// One workgroup of four waves per (path item, kv head).  The item holds up to
// 16 rows (its queries x the G query heads of the kv head) in one 16-row MFMA
// tile and a list of 32-token steps, each from one shared segment and seen by
// the queries in its mask.  Wave w takes steps w, w + 4, ...; each wave has
// two K/V slots of its own in LDS, filled by global_load_lds_dwordx4 one step
// ahead of the step it computes, so the waves never wait for each other until
// the end.  Per step: S^T = K Q^T (v_mfma_f32_16x16x32_bf16; A = K rows from
// LDS, B = the tile's Q in registers), the masked online softmax, and
// O^T += V^T P^T (V^T from the transposing LDS read), with the row sums from
// the same product against a tile of ones.  At the end the four waves' states
// and the queries' partial states from the MFMA items over the shared
// segments are merged by log-sum-exp and written as out / lse.
#include <hip/hip_ext.h>
#include <math.h>

#include "../kernels.hpp"
#include "common.hpp"
#include "tile.hpp"

namespace pkv {
namespace {

constexpr int kPathWaves = 4;
constexpr int kPathSlots = 2;        // K/V slots per wave
constexpr float kPathLoShare = 16.f; // residual term while a weight exceeds sum / 16

template <int D>
struct PathFin {
  float o[kPathWaves][16][D + 4];
  float m[kPathWaves][16];
  float l[kPathWaves][16];
  float wgt[16][kPathWaves + kMergeInline];   // normalised weights of each row's states
  int32_t prow[16][kMergeInline];             // partial rows (+ query head) of each row
  int32_t np[16];
};
template <int D>
union PathSmem {
  char slot[kPathWaves][kPathSlots][2][kStep * D * 2];   // [wave][slot][K, V]
  PathFin<D> fin;
};

template <int D>
__global__ __launch_bounds__(64 * kPathWaves) void path_kernel(const PathItem* __restrict__ items,
                                                              const PathStep* __restrict__ steps,
                                                              AttnParams p) {
  constexpr int NK = D / 32;
  constexpr int ND = D / 16;
  constexpr int CPR = D / 8;
  constexpr int RUNS = kStep * CPR / 64;   // 1 KB runs per K (or V) tile
  __shared__ PathSmem<D> sm;

  const int h = static_cast<int>(blockIdx.x);
  const int item = static_cast<int>(blockIdx.y);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int G = p.G;
  const PathItem& it = items[item];
  const int n_steps = it.n_steps;
  const int step0 = it.step_off;
  const int R = it.n_q * G;

  // the tile's row l16: query l16 / G, head l16 % G of this kv head
  const int my_q = l16 / G;
  const bool row_ok = l16 < R;
  bf16x8 qf[NK];
  {
    const int qi = row_ok ? it.q_index[my_q] : it.q_index[0];
    const uint16_t* qrow = p.q + (static_cast<size_t>(qi) * p.Hq + h * G + (row_ok ? l16 % G : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qrow + 32 * kk + 8 * g4);
    if (!row_ok) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) qf[kk] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  const uint4* kb = layer_head_base(p, p.k_pool, h, D);
  const uint4* vb = layer_head_base(p, p.v_pool, h, D);
  const uint32_t blk_chunks = static_cast<uint32_t>(p.Hkv * p.B * D / 8);
  const int bmask = p.B - 1;
  const int mine = wave < n_steps ? (n_steps - 1 - wave) / kPathWaves + 1 : 0;   // this wave's steps

  // step k of this wave (item step wave + 4 k) into slot k % 2: run u (K runs
  // first, then V) fills chunk slot c = 64 (u % RUNS) + lane of its tile,
  // row c / CPR, chunk (c % CPR) ^ tile_swz(row).  Tokens past the step's
  // count re-read its last token (masked below), so every run stays in the
  // pool.
  auto issue = [&](int k) __attribute__((always_inline)) {
    const PathStep ps = steps[step0 + wave + kPathWaves * k];
    const int off = ps.meta & 0xFF;
    const int last = ((ps.meta >> 8) & 0xFF) - 1;
    char* dst = sm.slot[wave][k % kPathSlots][0];
#pragma unroll
    for (int u = 0; u < 2 * RUNS; ++u) {
      const int c = (u % RUNS) * 64 + lane;
      const int r = c / CPR;
      const int ch = (c % CPR) ^ tile_swz<D>(r);
      const int t = min(r, last);
      const int blk = t < 16 ? ps.blk_a : ps.blk_b;
      const uint32_t ci = chunk_index(blk, blk_chunks, ((off + t) & bmask) * CPR + ch);
      lds_dma16((u < RUNS ? kb : vb) + ci, dst + (u >= RUNS ? kStep * D * 2 : 0) + (u % RUNS) * 1024);
    }
  };

  float m_run = -INFINITY;
  f32x4 o[ND + 1];   // o[ND]: row sums (P V against a tile of ones)
#pragma unroll
  for (int dt = 0; dt <= ND; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x8 ones = {0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80};

  if (mine > 0) issue(0);
  if (mine > 1) issue(1);
  // the query operands were loaded first: the compiler's wait for them lands here
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) asm volatile("" : "+v"(qf[kk]));
  for (int k = 0; k < mine; ++k) {
    // step k's runs have landed once only step k + 1's (2 RUNS) may be in flight
    if (k + 1 < mine)
      wait_vmcnt<2 * RUNS>();
    else
      wait_vmcnt<0>();
    const PathStep ps = steps[step0 + wave + kPathWaves * k];
    const int n_tok = (ps.meta >> 8) & 0xFF;
    const bool vis_row = row_ok && ((ps.qmask >> my_q) & 1u);
    const char* kt = sm.slot[wave][k % kPathSlots][0];
    const char* vt = kt + kStep * D * 2;
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + tile_byte<D>(16 * tt + l16, 4 * kk + g4));
        sacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[kk], sacc[tt], 0, 0, 0);
      }
    // each lane holds keys 16 tt + 4 g4 + i of its row l16
    float sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tok = 16 * (e >> 2) + 4 * g4 + (e & 3);
      sv[e] = (vis_row && tok < n_tok) ? sacc[e >> 2][e & 3] : -INFINITY;
    }
    float m = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) m = fmaxf(m, sv[e]);
    const float mx = xor32_max(xor16_max(m)) * p.scale_log2;
    // the reference max moves only when the row's max passes it by more than
    // kSlack (to that max): P <= 2^kSlack, the O rescale is rare
    const float m_new = mx > m_run + kSlack ? mx : m_run;
    if (__ballot(m_new != m_run)) {
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
#pragma unroll
      for (int dt = 0; dt <= ND; ++dt) o[dt] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float pv[8];
    uint32_t ph[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(fmaf(sv[e], p.scale_log2, -m_use));
#pragma unroll
    for (int e = 0; e < 8; e += 2) ph[e >> 1] = pack_bf16x2(pv[e], pv[e + 1]);
    uint4 hv = make_uint4(ph[0], ph[1], ph[2], ph[3]);
    const bf16x8 pf = *reinterpret_cast<bf16x8*>(&hv);
    // the row's largest weight of this step against its sum over the steps before
    const float p_top = mx == -INFINITY ? 0.f : fast_exp2(mx - m_use);
    const bool need_lo = __ballot(vis_row && p_top * kPathLoShare > o[ND][0]) != 0;
    auto vop = [&](int dt) __attribute__((always_inline)) {
      const int r = 4 * g4 + (l16 >> 2);
      const int c = 2 * dt + ((l16 & 3) >> 1);
      const int off = (l16 & 1) * 8;
      const v4i16 vlo = lds_read_tr16(vt + tile_byte<D>(r, c) + off);
      const v4i16 vhi = lds_read_tr16(vt + tile_byte<D>(16 + r, c) + off);
      return bf16x8{vlo[0], vlo[1], vlo[2], vlo[3], vhi[0], vhi[1], vhi[2], vhi[3]};
    };
#pragma unroll
    for (int dt = 0; dt <= ND; ++dt)
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dt < ND ? vop(dt) : ones, pf, o[dt], 0, 0, 0);
    if (need_lo) {
      uint32_t pl[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        pl[e >> 1] = pack_bf16x2(pv[e] - __uint_as_float(ph[e >> 1] << 16),
                                 pv[e + 1] - __uint_as_float(ph[e >> 1] & 0xFFFF0000u));
      uint4 lv = make_uint4(pl[0], pl[1], pl[2], pl[3]);
      const bf16x8 pfl = *reinterpret_cast<bf16x8*>(&lv);
#pragma unroll
      for (int dt = 0; dt <= ND; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dt < ND ? vop(dt) : ones, pfl, o[dt], 0, 0, 0);
    }
    // the slot's reads are done (their products consumed them): refill it
    if (k + 2 < mine) issue(k + 2);
  }
  wait_vmcnt<0>();

  // ---- merge: the four waves' states, then the queries' partial states ----
  lds_barrier();   // every wave is done with its slots (aliased below)
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
    *reinterpret_cast<float4*>(&sm.fin.o[wave][l16][16 * dt + 4 * g4]) =
        make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
  if (g4 == 0) {
    sm.fin.m[wave][l16] = m_run;
    sm.fin.l[wave][l16] = o[ND][0];
  }
  lds_barrier();
  // one thread per row: the common max and every state's normalised weight
  // (the partial states' lse loads leave together)
  if (tid < R) {
    const int row = tid;
    const int j = row / G;
    const int hq = h * G + row % G;
    const int mi = it.merge[j];
    const int np = mi >= 0 ? p.merges[mi].n_parts : 0;
    float lk[kMergeInline];
    int32_t pr[kMergeInline];
#pragma unroll
    for (int k = 0; k < kMergeInline; ++k) {
      pr[k] = k < np ? p.merges[mi].inl[k] + hq : 0;
      lk[k] = k < np ? p.part_lse[pr[k]] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kPathWaves; ++w)
      if (sm.fin.l[w][row] > 0.f) mx = fmaxf(mx, sm.fin.m[w][row]);
#pragma unroll
    for (int k = 0; k < kMergeInline; ++k) mx = fmaxf(mx, lk[k]);
    float aw[kPathWaves], ak[kMergeInline];
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kPathWaves; ++w) {
      const float lw = sm.fin.l[w][row];
      aw[w] = lw > 0.f ? fast_exp2(sm.fin.m[w][row] - mx) : 0.f;
      l = fmaf(aw[w], lw, l);
    }
#pragma unroll
    for (int k = 0; k < kMergeInline; ++k) {
      ak[k] = lk[k] == -INFINITY ? 0.f : fast_exp2(lk[k] - mx);
      l += ak[k];
    }
    const float inv = 1.f / l;
#pragma unroll
    for (int w = 0; w < kPathWaves; ++w) sm.fin.wgt[row][w] = aw[w] * inv;
#pragma unroll
    for (int k = 0; k < kMergeInline; ++k) {
      sm.fin.wgt[row][kPathWaves + k] = ak[k] * inv;
      sm.fin.prow[row][k] = pr[k];
    }
    sm.fin.np[row] = np;
    const size_t orow = static_cast<size_t>(it.q_index[j]) * p.Hq + hq;
    if (p.lse) p.lse[orow] = (mx + log2f(l)) * kLn2;
  }
  lds_barrier();
  // four consecutive dims of one row per thread and pass; the partial rows'
  // loads of a pass leave together
  constexpr int Q4 = D / 4;
  for (int u = tid; u < R * Q4; u += 64 * kPathWaves) {
    const int row = u / Q4;
    const int c = (u % Q4) * 4;
    const int np = sm.fin.np[row];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kPathWaves; ++w) {
      const float a = sm.fin.wgt[row][w];
      const float4 x = *reinterpret_cast<const float4*>(&sm.fin.o[w][row][c]);
      acc.x = fmaf(a, x.x, acc.x);
      acc.y = fmaf(a, x.y, acc.y);
      acc.z = fmaf(a, x.z, acc.z);
      acc.w = fmaf(a, x.w, acc.w);
    }
    if (np > 0) {
      float4 x[kMergeInline];
#pragma unroll
      for (int k = 0; k < kMergeInline; ++k)
        x[k] = *reinterpret_cast<const float4*>(p.part_o + static_cast<size_t>(sm.fin.prow[row][k < np ? k : 0]) * D + c);
#pragma unroll
      for (int k = 0; k < kMergeInline; ++k) {
        const float a = k < np ? sm.fin.wgt[row][kPathWaves + k] : 0.f;
        acc.x = fmaf(a, x[k].x, acc.x);
        acc.y = fmaf(a, x[k].y, acc.y);
        acc.z = fmaf(a, x[k].z, acc.z);
        acc.w = fmaf(a, x[k].w, acc.w);
      }
    }
    const size_t orow = static_cast<size_t>(it.q_index[row / G]) * p.Hq + h * G + row % G;
    *reinterpret_cast<float4*>(p.out + orow * D + c) = acc;
  }
}

}  // namespace

hipError_t launch_path(const AttnParams& p, const PathItem* items, int32_t n_items, int32_t head_dim,
                       hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (n_items == 0) return hipSuccess;
  if (n_items > 65535 || p.G > 16 || p.B < 16) return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>(p.Hkv), static_cast<uint32_t>(n_items));
  if (head_dim == 64)
    hipExtLaunchKernelGGL((path_kernel<64>), grid, dim3(64 * kPathWaves), 0, s, ev_start, ev_stop, 0, items,
                          p.steps, p);
  else if (head_dim == 128)
    hipExtLaunchKernelGGL((path_kernel<128>), grid, dim3(64 * kPathWaves), 0, s, ev_start, ev_stop, 0, items,
                          p.steps, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
