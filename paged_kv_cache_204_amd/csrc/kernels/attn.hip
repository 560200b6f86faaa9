// Paged attention over the block pool: one launch per call.
//
// Each workgroup (256 or 512 threads) runs one work item of the plan for one
// kv head -- a run of key tokens reached through the block table and up to
// a tile of query rows (row groups x the G query heads of this kv head):
//
//  * MFMA items (the first n_mfma): the query tile is a real dense
//    contraction -- every node of a draft tree (CAST page, technical
//    summary "Problem": the target checks the whole tree in one pass) or a
//    shared prefix under many queries.  W (4 or 8) waves x RT row tiles of
//    16 rows.
//  * VALU items: one decode query's GQA group (or two); up to 8 rows.
//
// Decode is bound by memory bandwidth (SGLang RadixAttention page, section on
// the KV-cache lifecycle): K/V move with 128-bit loads whose addresses come
// from the block table staged in LDS, loads are unconditional (tokens past
// the end re-read the last token and are masked) and barriers order LDS only,
// so loads issued ahead stay in flight.
//
// Items that cover only part of a query's keys write a normalised partial
// state (o, base-2 lse) that the merge launch combines.  (Merging inside
// this launch would need device-scope release/acquire fences per workgroup;
// on this GPU those write back and invalidate the whole L2 of an XCD, which
// costs far more than a second launch and evicts shared blocks.)
#include <hip/hip_ext.h>
#include <math.h>

#include <type_traits>

#include "../kernels.hpp"
#include "common.hpp"
#include "tile.hpp"

namespace pkv {
namespace {

constexpr int kThreads = 256;

constexpr int kBufs = 3;           // tiles in LDS: the step being read, the next two landing
template <int D>
struct MfmaSmem {
  char k[kBufs][kStep * D * 2];
  char v[kBufs][kStep * D * 2];
};

// One 32-token step of the MFMA path for the RT row tiles of one wave:
// S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = K rows, B = Q rows in
// registers), the masked online softmax, and O^T += V^T P^T.  kop(tt, kk)
// gives the K operand of tokens 16 tt + l16, dims 32 kk + 8 g4 .. + 7;
// vop(dt) the V^T operand of dim 16 dt + l16, tokens 4 g4 .. + 3 and
// 16 + 4 g4 .. + 3; after_qk() runs once the score products are issued.  The score accumulator gives each lane
// 4 tokens of ONE query row (row l16, tokens 16 tt + 4 g4 + i), so the
// softmax max / sum need two cross-row swaps only, and the rounded P (bf16)
// of the lane's 8 tokens is exactly the B operand of the P V product.  O^T
// keeps each lane on the same row, so the online rescale is lane local; it
// runs only when some row of the wave outgrows its reference max by more
// than kSlack.
template <int D, int RT, class KOp, class VOp, class AfterQK>
__device__ __forceinline__ void mfma_tile(KOp kop, VOp vop, AfterQK after_qk,
                                          const bf16x8 (&qf)[RT][D / 32], const uint64_t (&anc)[RT],
                                          const WorkItem& it, int t0, float scale_log2,
                                          float (&m_run)[RT], float (&l_run)[RT],
                                          f32x4 (&o)[RT][D / 16]) {
  constexpr int NK = D / 32;
  constexpr int ND = D / 16;
  const int g4 = (threadIdx.x & 63) >> 4;
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
      const bf16x8 a = kop(tt, kk);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        sacc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[rt][kk], sacc[rt][tt], 0, 0, 0);
    }
  }
  after_qk();
  const bool full = t0 + kStep <= it.n_tok && t0 + kStep <= it.tail_start;
  bf16x8 pf[RT], pf_lo[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float sv[8];   // raw scores; the scale is applied inside the exponent
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[4 * tt + i] = sacc[rt][tt][i];
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
    mx = xor32_max(xor16_max(mx)) * scale_log2;
    // The reference max m moves only when a row's max passes it by more
    // than kSlack (then the whole wave rescales, every row to its exact
    // max), so P <= 2^kSlack and the O rescale is rare after the first
    // steps.  P enters the PV product as two bf16 terms, hi = bf16(P) and
    // lo = bf16(P - hi), which carry it to about 2^-17 relative: a single
    // bf16 P would leave up to 2^-9 relative error on each weight, which
    // on rows of a few keys reaches 4e-3 in the output.
    const float m_old = m_run[rt];
    if (__ballot(mx > m_old + kSlack)) {
      const float m_new = fmaxf(mx, m_old);
      const float alpha = (m_old == -INFINITY) ? 0.f : fast_exp2(m_old - m_new);
      l_run[rt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) o[rt][dt] *= alpha;
      m_run[rt] = m_new;
    }
    const float m_use = (m_run[rt] == -INFINITY) ? 0.f : m_run[rt];
    float ps = 0.f;
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const float p0 = fast_exp2(fmaf(sv[j], scale_log2, -m_use));
      const float p1 = fast_exp2(fmaf(sv[j + 1], scale_log2, -m_use));
      ps += p0 + p1;
      const uint32_t h = pack_bf16x2(p0, p1);
      ph[j >> 1] = h;
      pl[j >> 1] = pack_bf16x2(p0 - __uint_as_float(h << 16), p1 - __uint_as_float(h & 0xFFFF0000u));
    }
    l_run[rt] += ps;
    uint4 hv = make_uint4(ph[0], ph[1], ph[2], ph[3]);
    uint4 lv = make_uint4(pl[0], pl[1], pl[2], pl[3]);
    pf[rt] = *reinterpret_cast<bf16x8*>(&hv);
    pf_lo[rt] = *reinterpret_cast<bf16x8*>(&lv);
  }
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) {
    const bf16x8 a = vop(dt);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[rt], o[rt][dt], 0, 0, 0);
      o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf_lo[rt], o[rt][dt], 0, 0, 0);
    }
  }
}

// One MFMA work item.  The K and V tiles of each 32-token step go from global
// memory straight into LDS (global_load_lds_dwordx4: lane i of one
// instruction fills bytes 16 i .. 16 i + 15 of a 1 KB run), two steps ahead
// into a ring of three tiles, so no registers hold them and no instructions
// repack them; every wave then runs mfma_tile on its own RT row tiles, with
// V^T read through the transposing LDS read.
template <int D, int RT, int W>
__device__ __forceinline__ void mfma_item(const AttnParams& p, const WorkItem& it, int h,
                                          MfmaSmem<D>& sm, const int32_t* blk_s) {
  constexpr int NK = D / 32;
  constexpr int ND = D / 16;
  constexpr int CPR = D / 8;
  constexpr int RUNS = kStep * CPR / 64;    // 1 KB runs per tile
  constexpr int IPW = 2 * RUNS / W;         // K and V runs each wave loads per step
  static_assert(IPW * W == 2 * RUNS, "a step's runs split evenly over the waves");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int G = p.G;
  const int R = it.n_grp * G;

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
      const RowOf ro = row_of(p, r);
      const RowGroup g = p.groups[it.grp_off + ro.grp];
      const int hq = h * G + ro.head;
      const uint16_t* qrow = p.q + (static_cast<size_t>(g.q_index) * p.Hq + hq) * D;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        qf[rt][kk] = *reinterpret_cast<const bf16x8*>(qrow + 32 * kk + 8 * g4);
      anc[rt] = (static_cast<uint64_t>(g.anc_hi) << 32) | g.anc_lo;
      dst_row[rt] = it.part_base < 0
                        ? static_cast<size_t>(g.q_index) * p.Hq + hq
                        : static_cast<size_t>(it.part_base) + static_cast<size_t>(ro.grp) * p.Hq + hq;
    }
  }
  const bool active = wave * RT * 16 < R;

  float m_run[RT], l_run[RT];
  f32x4 o[RT][ND];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const uint4* kb = layer_head_base(p, p.k_pool, h, D);
  const uint4* vb = layer_head_base(p, p.v_pool, h, D);
  const uint32_t blk_chunks = static_cast<uint32_t>(p.Hkv * p.B * D / 8);
  const int t_last = it.n_tok - 1;
  // Run j of a step (K runs first, then V): lane i fills chunk slot
  // q = 64 (j % RUNS) + i of its tile, i.e. row q / CPR and chunk
  // (q % CPR) ^ tile_swz(row).  Tokens past the end re-read the last token
  // (masked in the softmax), so every run stays inside the pool.
  auto issue = [&](int s) {
    const int t0 = s * kStep;
    const int b = s % kBufs;
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      const int j = wave * IPW + u;
      const int q = (j % RUNS) * 64 + lane;
      const int r = q / CPR;
      const int c = (q % CPR) ^ tile_swz<D>(r);
      const int t = min(t0 + r, t_last);
      const uint32_t ci = chunk_index(blk_s[t >> p.log2B], blk_chunks, (t & (p.B - 1)) * CPR + c);
      char* dst = (j >= RUNS ? sm.v[b] : sm.k[b]) + (j % RUNS) * 1024;
      lds_dma16((j >= RUNS ? vb : kb) + ci, dst);
    }
  };
  const int nsteps = (it.n_tok + kStep - 1) / kStep;

  issue(0);
  issue(1);
  // The query operands and masks were loaded first; taking them here makes
  // the compiler's wait for them (which also drains the first two steps'
  // runs, younger in the in-order count) land before the loop, not at their
  // first use inside it, where it would drain every step's runs.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) asm volatile("" : "+v"(qf[rt][kk]));
    asm volatile("" : "+v"(anc[rt]));
  }
  for (int s = 0; s < nsteps; ++s) {
    // this wave's runs of step s have landed (those of step s + 1 may still
    // be in flight); the barrier shows every wave's runs to all, and orders
    // the reads of the tile that step s + 2 overwrites before its runs
    wait_vmcnt<IPW>();
    lds_barrier();
    issue(s + 2);
    if (!active) continue;
    const char* kt = sm.k[s % kBufs];
    const char* vt = sm.v[s % kBufs];
    const auto kop = [&](int tt, int kk) {
      return *reinterpret_cast<const bf16x8*>(kt + tile_byte<D>(16 * tt + l16, 4 * kk + g4));
    };
    // lane (l16, g4) of a 16-lane group names 4 dims of one token row; the
    // transposed read hands lane i of the group dim 16 dt + i of 4 tokens
    const auto vop = [&](int dt) {
      const int r = 4 * g4 + (l16 >> 2);
      const int c = 2 * dt + ((l16 & 3) >> 1);
      const int off = (l16 & 1) * 8;
      const v4i16 lo = lds_read_tr16(vt + tile_byte<D>(r, c) + off);
      const v4i16 hi = lds_read_tr16(vt + tile_byte<D>(16 + r, c) + off);
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    mfma_tile<D, RT>(kop, vop, [] {}, qf, anc, it, s * kStep, p.scale_log2, m_run, l_run, o);
  }
  // the runs issued past the last step land before the workgroup ends
  wait_vmcnt<0>();

  if (!active) return;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float l = xor32_sum(xor16_sum(l_run[rt]));
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

// ---------------------------------------------------------------- VALU path
constexpr int kValuRows = kValuMaxRows;
constexpr int kValuTok = kValuMaxTokens;
constexpr int kTokPerRound = 128;  // K tokens with loads in flight per workgroup
constexpr int kUnrollV = 8;        // V tokens in flight per lane

template <int D>
struct alignas(16) ValuSmem {
  float s[kValuTok][kValuRows];   // scores, then probabilities, token-major
  float red[kThreads / 64][4][D]; // per-wave P V sums (one-row-per-wave items)
  float m[kValuRows], l[kValuRows];
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot8(const uint4& q, const uint4& k, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.x), __builtin_bit_cast(bf16x2_t, k.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.y), __builtin_bit_cast(bf16x2_t, k.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.z), __builtin_bit_cast(bf16x2_t, k.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w), __builtin_bit_cast(bf16x2_t, k.w), acc, false);
  return acc;
}


// Phase 3 for items of one row per wave (RM = 4): the waves split the
// tokens, each lane accumulates all rows for its 8 dims, a butterfly over
// the token slots and a sum over the waves through LDS give O.
template <int D, int RM, class Addr, class VTok>
__device__ __forceinline__ void valu_pv_split(const AttnParams& p, const WorkItem& it, int h,
                                              ValuSmem<D>& sm, uint4 (&vv)[kUnrollV], const uint4* vb,
                                              Addr addr, VTok vtok, int nv, const int32_t* qidx) {
  constexpr int CPR = D / 8;
  static_assert(RM == 4, "one row per wave");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = tid % CPR;
  const int ts = lane / CPR;
  const int t_last = it.n_tok - 1;
  const int R = it.n_grp * p.G;
  float o[RM][8];
#pragma unroll
  for (int r = 0; r < RM; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[r][e] = 0.f;
  for (int k0 = 0; k0 < nv; k0 += kUnrollV) {
    if (k0 > 0) {
#pragma unroll
      for (int u = 0; u < kUnrollV; ++u) vv[u] = vb[addr(vtok(k0 + u))];
    }
#pragma unroll
    for (int u = 0; u < kUnrollV; ++u) {
      const int t = vtok(k0 + u);
      float4 pr = *reinterpret_cast<const float4*>(&sm.s[min(t, t_last)][0]);
      if (t > t_last) pr = make_float4(0.f, 0.f, 0.f, 0.f);
      const float pa[4] = {pr.x, pr.y, pr.z, pr.w};
      const float v[8] = {bf16_lo(vv[u].x), bf16_hi(vv[u].x), bf16_lo(vv[u].y), bf16_hi(vv[u].y),
                          bf16_lo(vv[u].z), bf16_hi(vv[u].z), bf16_lo(vv[u].w), bf16_hi(vv[u].w)};
#pragma unroll
      for (int r = 0; r < RM; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[r][e] = fmaf(pa[r], v[e], o[r][e]);
    }
  }
#pragma unroll
  for (int r = 0; r < RM; ++r) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = o[r][e];
      if constexpr (CPR == 8) x += dpp_f32<kDppXor8>(x);
      o[r][e] = xor32_sum(xor16_sum(x));
    }
  }
  if (ts == 0) {
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      *reinterpret_cast<float4*>(&sm.red[wave][r][c * 8]) = make_float4(o[r][0], o[r][1], o[r][2], o[r][3]);
      *reinterpret_cast<float4*>(&sm.red[wave][r][c * 8 + 4]) = make_float4(o[r][4], o[r][5], o[r][6], o[r][7]);
    }
  }
  lds_barrier();
  constexpr int kQuads = D / 4;
  for (int e = tid; e < R * kQuads; e += kThreads) {
    const int r = e / kQuads;
    const int d = (e % kQuads) * 4;
    float4 acc = *reinterpret_cast<const float4*>(&sm.red[0][r][d]);
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) {
      const float4 x = *reinterpret_cast<const float4*>(&sm.red[w][r][d]);
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
    const float l = sm.l[r];
    const float m = sm.m[r];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const RowOf ro = row_of(p, r);
    const int hq = h * p.G + ro.head;
    const float4 val = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    if (it.part_base < 0) {
      const size_t row = static_cast<size_t>(qidx[ro.grp]) * p.Hq + hq;
      *reinterpret_cast<float4*>(p.out + row * D + d) = val;
      if (p.lse && d == 0) p.lse[row] = (m + log2f(l)) * kLn2;
    } else {
      const size_t row = static_cast<size_t>(it.part_base) + static_cast<size_t>(ro.grp) * p.Hq + hq;
      *reinterpret_cast<float4*>(p.part_o + row * D + d) = val;
      if (d == 0) p.part_lse[row] = l > 0.f ? m + log2f(l) : -INFINITY;
    }
  }
}

// Phase 1 (whole workgroup): a token's head_dim row is read by D/8 lanes
// with 128-bit loads (the row is one coalesced burst); each lane forms the
// partial dot products of every row over its 8 dims (v_dot2_f32_bf16), a
// DPP butterfly over the token's lanes completes them, and the scores land
// in LDS token-major.  One workgroup barrier.  Phase 2 (each wave alone,
// RM / 4 rows per wave): exact softmax of the wave's rows over the item's
// keys.  Phase 3, O = P V with lane = (8-dim chunk, token slot), the V
// chunks of a lane's first tokens requested before phase 1:
//  * RM = 8 (two rows per wave): each wave walks all tokens for its own
//    rows, reading the rows' P pair of a token with one 64-bit LDS read; a
//    butterfly over the token slots sums O, with no further barrier;
//  * RM = 4 (one row per wave): the waves split the tokens instead and
//    every lane keeps all four rows (valu_pv_split), so each V row is
//    loaded once per workgroup; O is summed over slots and waves.
// RM bounds the rows at compile time; rows >= R are never written.
template <int D, int RM>
__device__ __forceinline__ void valu_item(const AttnParams& p, const WorkItem& it, int item, int h,
                                          ValuSmem<D>& sm, const int32_t* blk_s) {
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int TPP = kThreads / CPR;
  constexpr int TS = 64 / CPR;      // token slots of a wave in phase 3
  constexpr int RW = RM / 4;        // rows per wave in phase 2 (and phase 3 when 2)
  constexpr int kUnroll = kTokPerRound / TPP;   // K passes with loads in flight
  static_assert(RM <= CPR, "one score row per lane of a token group");
  static_assert(RW == 1 || RW == 2, "one or two rows per wave");
  const int G = p.G;
  const int R = it.n_grp * G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = tid % CPR;
  const int tp = tid / CPR;
  const int ts = lane / CPR;
  const int r0 = wave * RW;
  // read from the item in memory (uniform loads), not from its register copy
  const int32_t* qidx = p.items[item].q_index;

  const uint4* kb = layer_head_base(p, p.k_pool, h, D);
  const uint4* vb = layer_head_base(p, p.v_pool, h, D);
  const uint32_t blk_chunks = static_cast<uint32_t>(p.Hkv * p.B * D / 8);
  const int t_last = it.n_tok - 1;
  auto addr = [&](int t) {
    t = min(t, t_last);
    return chunk_index(blk_s[t >> p.log2B], blk_chunks, (t & (p.B - 1)) * (D / 8) + c);
  };
  const int npass = (it.n_tok + TPP - 1) / TPP;
  // Phase-3 token k of a lane: with two rows per wave every wave walks all
  // tokens (slot ts of each TS); with one row per wave the waves split the
  // tokens (wave w takes every fourth group of TS) and sum through LDS.
  auto vtok = [&](int k) { return RW == 2 ? ts + TS * k : ts + TS * (wave + 4 * k); };
  const int nv = RW == 2 ? (it.n_tok + TS - 1) / TS : (it.n_tok + 4 * TS - 1) / (4 * TS);

  // first K passes, first V tokens of this lane, then the queries
  uint4 kv[kUnroll], vv[kUnrollV];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) kv[u] = kb[addr(u * TPP + tp)];
#pragma unroll
  for (int u = 0; u < kUnrollV; ++u) vv[u] = vb[addr(vtok(u))];
  uint4 qv[RM];
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    qv[r] = make_uint4(0, 0, 0, 0);
    if (r < R) {
      const RowOf ro = row_of(p, r);
      const size_t qoff = (static_cast<size_t>(qidx[ro.grp]) * p.Hq + h * G + ro.head) * D + c * 8;
      qv[r] = *reinterpret_cast<const uint4*>(p.q + qoff);
    }
  }
  uint64_t anc_mine = 0;
  if (c < R) {
    const RowGroup g = p.groups[it.grp_off + row_of(p, c).grp];
    anc_mine = (static_cast<uint64_t>(g.anc_hi) << 32) | g.anc_lo;
  }

  // ---- phase 1: scores ---------------------------------------------------
  for (int p0 = 0; p0 < npass; p0 += kUnroll) {
    if (p0 > 0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) kv[u] = kb[addr((p0 + u) * TPP + tp)];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = (p0 + u) * TPP + tp;
      float mine = 0.f;
#pragma unroll
      for (int r = 0; r < RM; ++r) {
        const float sr = group_sum<CPR>(dot8(qv[r], kv[u], 0.f));
        mine = (r == c) ? sr : mine;
      }
      if (c < R && t < it.n_tok) {
        bool vis = true;
        if (t >= it.tail_start) vis = (anc_mine >> (it.tail_node0 + t - it.tail_start)) & 1ull;
        sm.s[t][c] = vis ? mine * p.scale_log2 : -INFINITY;
      }
    }
  }
  lds_barrier();
  if (RW == 2 && r0 >= R) return;   // no workgroup barrier follows on this path

  // ---- phase 2: exact softmax of this wave's rows --------------------------
  // The wave's rows go through together (their reductions interleave); a
  // row past R (odd G only) computes on unused LDS and is never stored.
  float m_row[RW], l_row[RW];
  {
    float mx[RW], sum[RW];
#pragma unroll
    for (int j = 0; j < RW; ++j) mx[j] = -INFINITY;
    for (int t = lane; t < it.n_tok; t += 64) {
#pragma unroll
      for (int j = 0; j < RW; ++j) mx[j] = fmaxf(mx[j], sm.s[t][r0 + j]);
    }
    float m_use[RW];
#pragma unroll
    for (int j = 0; j < RW; ++j) {
      mx[j] = wave_max(mx[j]);
      m_use[j] = (mx[j] == -INFINITY) ? 0.f : mx[j];
      sum[j] = 0.f;
    }
    for (int t = lane; t < it.n_tok; t += 64) {
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        const float e = fast_exp2(sm.s[t][r0 + j] - m_use[j]);
        sm.s[t][r0 + j] = e;
        sum[j] += e;
      }
    }
#pragma unroll
    for (int j = 0; j < RW; ++j) {
      m_row[j] = mx[j];
      l_row[j] = wave_sum(sum[j]);
    }
  }
  if constexpr (RW == 1) {
    // phase 3 reads every row's P and the final step every row's m, l
    if (lane == 0) {
      sm.m[r0] = m_row[0];
      sm.l[r0] = l_row[0];
    }
    lds_barrier();
    valu_pv_split<D, RM>(p, it, h, sm, vv, vb, addr, vtok, nv, qidx);
    return;
  }
  wave_lds_sync();

  // ---- phase 3: O = P V for this wave's rows --------------------------------
  float o[RW][8];
#pragma unroll
  for (int j = 0; j < RW; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
  for (int k0 = 0; k0 < nv; k0 += kUnrollV) {
    if (k0 > 0) {
#pragma unroll
      for (int u = 0; u < kUnrollV; ++u) vv[u] = vb[addr(vtok(k0 + u))];
    }
#pragma unroll
    for (int u = 0; u < kUnrollV; ++u) {
      const int t = vtok(k0 + u);
      const int tc = min(t, t_last);
      float pr[RW];
      if constexpr (RW == 2) {
        const float2 a = *reinterpret_cast<const float2*>(&sm.s[tc][r0]);
        pr[0] = a.x;
        pr[1] = a.y;
      } else {
        pr[0] = sm.s[tc][r0];
      }
      if (t > t_last) {
#pragma unroll
        for (int j = 0; j < RW; ++j) pr[j] = 0.f;
      }
      const float v[8] = {bf16_lo(vv[u].x), bf16_hi(vv[u].x), bf16_lo(vv[u].y), bf16_hi(vv[u].y),
                          bf16_lo(vv[u].z), bf16_hi(vv[u].z), bf16_lo(vv[u].w), bf16_hi(vv[u].w)};
#pragma unroll
      for (int j = 0; j < RW; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] = fmaf(pr[j], v[e], o[j][e]);
    }
  }
  // sum over the token slots (lanes that hold the same dims)
#pragma unroll
  for (int j = 0; j < RW; ++j) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = o[j][e];
      if constexpr (CPR == 8) x += dpp_f32<kDppXor8>(x);
      o[j][e] = xor32_sum(xor16_sum(x));
    }
  }
  if (ts != 0) return;
#pragma unroll
  for (int j = 0; j < RW; ++j) {
    const int r = r0 + j;
    if (r >= R) continue;
    const float l = l_row[j];
    const float m = m_row[j];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const RowOf ro = row_of(p, r);
    const int hq = h * G + ro.head;
    const float4 lo = make_float4(o[j][0] * inv, o[j][1] * inv, o[j][2] * inv, o[j][3] * inv);
    const float4 hi = make_float4(o[j][4] * inv, o[j][5] * inv, o[j][6] * inv, o[j][7] * inv);
    float* dst;
    if (it.part_base < 0) {
      const size_t row = static_cast<size_t>(qidx[ro.grp]) * p.Hq + hq;
      dst = p.out + row * D + c * 8;
      if (p.lse && c == 0) p.lse[row] = (m + log2f(l)) * kLn2;
    } else {
      const size_t row = static_cast<size_t>(it.part_base) + static_cast<size_t>(ro.grp) * p.Hq + hq;
      dst = p.part_o + row * D + c * 8;
      if (c == 0) p.part_lse[row] = l > 0.f ? m + log2f(l) : -INFINITY;
    }
    *reinterpret_cast<float4*>(dst) = lo;
    *reinterpret_cast<float4*>(dst + 4) = hi;
  }
}

// The fields a workgroup needs first also come as leading scalar arguments:
// the build preloads leading kernel arguments into SGPRs, so the item, block
// list and query loads leave at wave start instead of after a kernel-argument
// fetch.
template <int D, int RT, int RM, int W>
__global__ __launch_bounds__(64 * W) void attn_kernel(const WorkItem* __restrict__ items,
                                                        const int32_t* __restrict__ blocks,
                                                        const RowGroup* __restrict__ groups,
                                                        const uint16_t* __restrict__ q,
                                                        int32_t n_mfma, int32_t stride_mfma,
                                                        int32_t stride_valu, AttnParams p) {
  p.items = items;
  p.blocks = blocks;
  p.groups = groups;
  p.q = q;
  p.n_mfma = n_mfma;
  p.stride_mfma = stride_mfma;
  p.stride_valu = stride_valu;
  __shared__ union alignas(16) {
    MfmaSmem<D> m;
    ValuSmem<D> v;
  } sm;
  __shared__ int32_t blk_s[kMaxItemBlocks];

  // Workgroup -> (item, kv head): the MFMA items of every head first, item
  // by item (the planner sorts each kind longest first), then the VALU
  // items, so the long items start early and the short ones fill in.
  const int L = static_cast<int>(blockIdx.x);
  const bool is_mfma = L < p.n_mfma * p.Hkv;
  const int wi = is_mfma ? L : L - p.n_mfma * p.Hkv;
  const int h = wi % p.Hkv;
  const int item = (is_mfma ? 0 : p.n_mfma) + wi / p.Hkv;
  // the block list sits at a stride fixed per item kind, so its loads go
  // out together with the item's
  const int nb = is_mfma ? p.stride_mfma : p.stride_valu;
  const int32_t* lst = p.blocks + (is_mfma ? static_cast<size_t>(item) * p.stride_mfma
                                           : static_cast<size_t>(p.n_mfma) * p.stride_mfma +
                                                 static_cast<size_t>(item - p.n_mfma) * p.stride_valu);
  for (int i = threadIdx.x; i < nb; i += 64 * W) blk_s[i] = lst[i];
  const WorkItem it = p.items[item];
  lds_barrier();
  if constexpr (W == 4) {
    if (is_mfma)
      mfma_item<D, RT, 4>(p, it, h, sm.m, blk_s);
    else
      valu_item<D, RM>(p, it, item, h, sm.v, blk_s);
  } else {
    // eight-wave workgroups serve launches whose items are all MFMA items
    mfma_item<D, RT, W>(p, it, h, sm.m, blk_s);
  }
}

// ---------------------------------------------------------------- direct path
// Decode calls of few, short queries: one workgroup per (query, kv head)
// covers all of the query's keys, so the call writes no partial states and
// needs no merge launch.  The W waves take the 32-token steps in turn (wave
// w the steps w, w + W, ...) and run mfma_tile on one 16-row tile that holds
// the query's G <= 16 heads (rows G..15 are zero).  No wave reads another's
// tile, so K goes from global memory straight into the lane's MFMA operand
// registers and V sits in an LDS region of the wave's own, read back
// transposed with ds_read_b64_tr_b16; only wave-level ordering is needed.
// Two forms: the rolling one stages V through registers into a row buffer
// and runs its loads DEPTH steps ahead; the one-round one (ALL, below)
// issues every load of the wave at once.  At the end the waves' softmax
// states (m, l, O) meet in LDS and are merged by log-sum-exp, one output
// element per lane.
template <int D, int W>
struct DirectFin {
  float o[W][16][D + 4];
  float m[W][16];
  float l[W][16];
};
template <int D, int W>
union DirectSmem {
  uint16_t v[W][kStep][D + 8];   // each wave's V rows, padded pitch
  DirectFin<D, W> fin;
};
// One-round form: every step of a wave has a V tile of its own (the
// swizzled layout of the MFMA path, filled by LDS DMA); the merge area is
// separate, so a wave stores its state without waiting for the others.
template <int D, int W, int S>
struct DirectSmemAll {
  char vt[W][S][kStep * D * 2];
  DirectFin<D, W> fin;
};
// The same with one V tile per step of the call (step s in tile s, at most
// NSLOT steps) under the merge area, which the waves fill after a barrier:
// less LDS, so two workgroups fit on a CU.
template <int D, int W, int NSLOT>
union DirectSmemSteps {
  char vt[NSLOT][kStep * D * 2];
  DirectFin<D, W> fin;
};

// The grid is (kv head, item), so a workgroup finds its item and head
// without arithmetic on kernel arguments, and the first loads (the item's
// block list, its WorkItem, the query rows) leave together at wave start:
// the block-list loads are unconditional (indexes clamped into the list)
// and come first in program order, the query row needs only the WorkItem.
// Everything the prologue and the K/V addressing read from the arguments
// sits in the first 14 dwords (hq; g and log2 of the block size packed in
// one dword; the block pitch in 16-byte chunks; the layer's K/V bases),
// which arrive preloaded in SGPRs, so no argument load stands in the chain.
// Only the K/V loads wait for the list, through LDS and one barrier.
//
// ALL (calls whose every wave has at most DEPTH steps): a wave issues the
// loads of all of its steps at once -- K into registers, then V by LDS DMA
// into DEPTH tiles of its own -- so the call waits for one memory round
// trip, not one per DEPTH steps; V then costs no registers.  NSLOT > 0
// (calls of at most NSLOT steps): the V tiles are indexed by step and a wave
// loads only the steps it computes.
//
// LAYERS: grid.z runs over consecutive layers of one call (the same items
// and block lists); workgroup z reads layer p.layer + z of the pools, its
// query rows and writes its out / lse rows at z times the layer's row count.
template <int D, int W, int DEPTH, bool ALL, bool LAYERS, int NSLOT = 0>
__global__ __launch_bounds__(64 * W) void direct_kernel(const WorkItem* __restrict__ items,
                                                          const int32_t* __restrict__ blocks,
                                                          const uint16_t* __restrict__ q,
                                                          int32_t stride, int32_t hq,
                                                          uint32_t g_log2B, uint32_t blk_chunks,
                                                          const uint4* __restrict__ k_layer,
                                                          const uint4* __restrict__ v_layer,
                                                          AttnParams p) {
  constexpr int NK = D / 32;
  constexpr int ND = D / 16;
  constexpr int CPR = D / 8;
  constexpr int VPER = kStep * CPR / 64;   // V chunks per lane per step
  constexpr int LPER = (kMaxItemBlocks + 64 * W - 1) / (64 * W);   // block-list entries per thread
  static_assert(VPER * 64 == kStep * CPR, "a step's V splits evenly over a wave");
  using Smem = std::conditional_t<ALL, std::conditional_t<(NSLOT > 0), DirectSmemSteps<D, W, NSLOT>, DirectSmemAll<D, W, DEPTH>>, DirectSmem<D, W>>;
  __shared__ Smem sm;
  __shared__ int32_t blk_s[kMaxItemBlocks];

  const int h = static_cast<int>(blockIdx.x);
  const int item = static_cast<int>(blockIdx.y);
  const int g = static_cast<int>(g_log2B & 0xFFu);
  const int log2B = static_cast<int>(g_log2B >> 8);
  const int tid = threadIdx.x;
  const int32_t* lst = blocks + static_cast<size_t>(item) * stride;
  int32_t blk_r[LPER];
#pragma unroll
  for (int k = 0; k < LPER; ++k) blk_r[k] = lst[min(tid + 64 * W * k, stride - 1)];
  // keep the list loads ahead of the WorkItem's (whose wait they need not share)
  __builtin_amdgcn_sched_barrier(0);
  const int n_tok = items[item].n_tok;
  const int q_index = items[item].q_index[0];
  const int bmask = (1 << log2B) - 1;
  float* out_rows = p.out;
  float* lse_rows = p.lse;
  if constexpr (LAYERS) {
    const size_t z = blockIdx.z;
    k_layer += z * p.layer_chunks;
    v_layer += z * p.layer_chunks;
    q += z * p.layer_rows * D;
    out_rows += z * p.layer_rows * D;
    if (lse_rows) lse_rows += z * p.layer_rows;
  }
  const uint4* kb = k_layer + ((static_cast<size_t>(h) * (D / 8)) << log2B);
  const uint4* vb = v_layer + ((static_cast<size_t>(h) * (D / 8)) << log2B);
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const size_t row0 = static_cast<size_t>(q_index) * hq + static_cast<size_t>(h) * g;

  bf16x8 qf[1][NK];
  {
    // rows past the group re-read row 0 of it and are zeroed after the load
    const uint16_t* qrow = q + (row0 + (l16 < g ? l16 : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) qf[0][kk] = *reinterpret_cast<const bf16x8*>(qrow + 32 * kk + 8 * g4);
  }
  // entries past the list repeat its last id and are never read
#pragma unroll
  for (int k = 0; k < LPER; ++k)
    if (64 * W * (k + 1) <= kMaxItemBlocks || tid + 64 * W * k < kMaxItemBlocks) blk_s[tid + 64 * W * k] = blk_r[k];
  if (l16 >= g) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) qf[0][kk] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
  WorkItem it{};
  it.n_tok = n_tok;
  it.tail_start = INT_MAX;
  const uint64_t anc[1] = {0};
  float m_run[1] = {-INFINITY}, l_run[1] = {0.f};
  f32x4 o[1][ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) o[0][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  lds_barrier();

  // K of token t0 + 16 tt + l16, chunk 4 kk + g4 is the lane's operand for
  // (tt, kk); V chunk ci = lane + 64 i is (token ci / CPR, chunk ci % CPR).
  // Tokens past the end re-read the last token (masked in the softmax).
  const int t_last = it.n_tok - 1;
  auto chunk_at = [&](int t, int c) {
    t = min(t, t_last);
    return chunk_index(blk_s[t >> log2B], blk_chunks, (t & bmask) * CPR + c);
  };
  auto ldg = [&](const uint4* src, int t, int c) { return src[chunk_at(t, c)]; };
  const int nsteps = (it.n_tok + kStep - 1) / kStep;
  const int mine = wave < nsteps ? (nsteps - 1 - wave) / W + 1 : 0;   // steps of this wave
  bf16x8 rk[DEPTH][2][NK];
  if constexpr (ALL) {
    // waves with the most steps set the workgroup's time: issue them first
    if (mine * W > nsteps) __builtin_amdgcn_s_setprio(2);
    // K of the wave's steps j = 0 .. DEPTH-1 (step wave + j W), then their V:
    // run u of step j's tile is lanes' chunk slots 64 u + lane, row q / CPR,
    // chunk (q % CPR) ^ tile_swz(row).  Steps past the wave's own re-read
    // the last token and are not computed.
#pragma unroll
    for (int j = 0; j < DEPTH; ++j)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
          rk[j][tt][kk] = __builtin_bit_cast(bf16x8, ldg(kb, (wave + j * W) * kStep + 16 * tt + l16, 4 * kk + g4));
    // (the sources are all looked up before the first copy: each copy is a
    // memory barrier to the compiler, which would otherwise wait for one
    // block-list read per copy)
    uint32_t vci[DEPTH][VPER];
#pragma unroll
    for (int j = 0; j < DEPTH; ++j)
#pragma unroll
      for (int u = 0; u < VPER; ++u) {
        const int q = 64 * u + lane;
        const int r = q / CPR;
        vci[j][u] = chunk_at((wave + j * W) * kStep + r, (q % CPR) ^ tile_swz<D>(r));
      }
    const int issued = NSLOT > 0 ? min(mine, DEPTH) : DEPTH;
    auto vtile = [&](int j) -> char* {
      if constexpr (NSLOT > 0) return sm.vt[wave + j * W]; else return sm.vt[wave][j];
    };
#pragma unroll
    for (int j = 0; j < DEPTH; ++j)
      if (NSLOT == 0 || j < issued)
#pragma unroll
        for (int u = 0; u < VPER; ++u) lds_dma16(vb + vci[j][u], vtile(j) + 1024 * u);
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      if (j >= mine) break;
      // step j's V runs have landed: only later steps' runs may be in flight
      wait_vmcnt_steps<VPER, DEPTH - 1>(issued - 1 - j);
      const char* vt = vtile(j);
      const auto kop = [&](int tt, int kk) { return rk[j][tt][kk]; };
      const auto vop = [&](int dt) {
        const int r = 4 * g4 + (l16 >> 2);
        const int c = 2 * dt + ((l16 & 3) >> 1);
        const int off = (l16 & 1) * 8;
        const v4i16 lo = lds_read_tr16(vt + tile_byte<D>(r, c) + off);
        const v4i16 hi = lds_read_tr16(vt + tile_byte<D>(16 + r, c) + off);
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      };
      mfma_tile<D, 1>(kop, vop, [] {}, qf, anc, it, (wave + j * W) * kStep, p.scale_log2, m_run, l_run, o);
    }
    // every run has landed before the tiles are reused for the merge
    wait_vmcnt<0>();
  } else {
  uint16_t (*vs)[D + 8] = sm.v[wave];
  uint4 rv[DEPTH][VPER];
  auto fetch = [&](int slot, int t0) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        rk[slot][tt][kk] = __builtin_bit_cast(bf16x8, ldg(kb, t0 + 16 * tt + l16, 4 * kk + g4));
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int ci = lane + 64 * i;
      rv[slot][i] = ldg(vb, t0 + ci / CPR, ci % CPR);
    }
  };
  auto step = [&](int slot, int s, bool prefetch) {
    // this wave's reads of its previous V tile are done before it is replaced
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int ci = lane + 64 * i;
      *reinterpret_cast<uint4*>(&vs[ci / CPR][(ci % CPR) * 8]) = rv[slot][i];
    }
    wave_lds_sync();
    const auto kop = [&](int tt, int kk) { return rk[slot][tt][kk]; };
    // lane (l16, g4) of each 16-lane group names 4 dims of one token row; the
    // transposed read hands lane i of the group dim 16 dt + i of 4 tokens
    const auto vop = [&](int dt) {
      const int r = 4 * g4 + (l16 >> 2);
      const int c = 16 * dt + 4 * (l16 & 3);
      const v4i16 lo = lds_read_tr16(&vs[r][c]);
      const v4i16 hi = lds_read_tr16(&vs[16 + r][c]);
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    // the slot's next loads leave once its K operands have been consumed
    const auto after_qk = [&] {
      if (prefetch) fetch(slot, (s + DEPTH * W) * kStep);
    };
    mfma_tile<D, 1>(kop, vop, after_qk, qf, anc, it, s * kStep, p.scale_log2, m_run, l_run, o);
  };

#pragma unroll
  for (int j = 0; j < DEPTH; ++j) fetch(j, (wave + j * W) * kStep);
  // whole rounds in which every step fetches the one DEPTH ahead, then the
  // last steps, of which only those with a step DEPTH ahead fetch
  int j0 = 0;
  for (; j0 + 2 * DEPTH <= mine; j0 += DEPTH) {
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) step(j, wave + (j0 + j) * W, true);
  }
#pragma unroll
  for (int j = 0; j < 2 * DEPTH - 1; ++j)
    if (j0 + j < mine) step(j % DEPTH, wave + (j0 + j) * W, j0 + j + DEPTH < mine);
  }

  // ---- merge of the W wave states ------------------------------------------
  const float l_w = xor32_sum(xor16_sum(l_run[0]));
  if constexpr (!ALL || NSLOT > 0) lds_barrier();   // every wave is done with its V region (aliased below)
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
    *reinterpret_cast<float4*>(&sm.fin.o[wave][l16][16 * dt + 4 * g4]) =
        make_float4(o[0][dt][0], o[0][dt][1], o[0][dt][2], o[0][dt][3]);
  if (g4 == 0) {
    sm.fin.m[wave][l16] = m_run[0];
    sm.fin.l[wave][l16] = l_w;
  }
  lds_barrier();
  // one output element per lane (G * D <= 16 * D elements over 64 W lanes)
  for (int e = tid; e < p.G * D; e += 64 * W) {
    const int row = e / D;
    const int c = e % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) mx = fmaxf(mx, sm.fin.m[w][row]);
    // wave 0 holds token 0, so mx is finite and l > 0
    float l = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = sm.fin.m[w][row];
      const float a = mw == -INFINITY ? 0.f : fast_exp2(mw - mx);
      l = fmaf(a, sm.fin.l[w][row], l);
      acc = fmaf(a, sm.fin.o[w][row][c], acc);
    }
    out_rows[(row0 + row) * D + c] = acc / l;
    if (c == 0 && lse_rows) lse_rows[row0 + row] = (mx + log2f(l)) * kLn2;
  }
}

}  // namespace

template <int D, int RT>
hipError_t launch_rows(const AttnParams& p, dim3 grid, int32_t valu_rows, int32_t waves, hipStream_t s,
                       hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (waves == 8) {
    if constexpr (RT == 2)
      hipExtLaunchKernelGGL((attn_kernel<D, RT, 4, 8>), grid, dim3(512), 0, s, ev_start, ev_stop, 0, p.items, p.blocks, p.groups,
                         p.q, p.n_mfma, p.stride_mfma, p.stride_valu, p);
    else
      return hipErrorInvalidValue;
  } else if (valu_rows <= 4) {
    hipExtLaunchKernelGGL((attn_kernel<D, RT, 4, 4>), grid, dim3(kThreads), 0, s, ev_start, ev_stop, 0, p.items, p.blocks, p.groups,
                       p.q, p.n_mfma, p.stride_mfma, p.stride_valu, p);
  } else {
    hipExtLaunchKernelGGL((attn_kernel<D, RT, 8, 4>), grid, dim3(kThreads), 0, s, ev_start, ev_stop, 0, p.items, p.blocks, p.groups,
                       p.q, p.n_mfma, p.stride_mfma, p.stride_valu, p);
  }
  return hipGetLastError();
}

hipError_t launch_attn(const AttnParams& p, int32_t n_items, int32_t head_dim, int32_t row_tiles,
                       int32_t valu_rows, int32_t waves, hipStream_t s, hipEvent_t ev_start,
                       hipEvent_t ev_stop) {
  if (n_items == 0) return hipSuccess;
  if (waves == 8 && n_items != p.n_mfma) return hipErrorInvalidValue;
  const int64_t n_wg = static_cast<int64_t>(n_items) * p.Hkv;
  if (n_wg > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>(n_wg));
  if (head_dim == 64 && row_tiles == 1) return launch_rows<64, 1>(p, grid, valu_rows, waves, s, ev_start, ev_stop);
  if (head_dim == 64 && row_tiles == 2) return launch_rows<64, 2>(p, grid, valu_rows, waves, s, ev_start, ev_stop);
  if (head_dim == 128 && row_tiles == 1) return launch_rows<128, 1>(p, grid, valu_rows, waves, s, ev_start, ev_stop);
  if (head_dim == 128 && row_tiles == 2) return launch_rows<128, 2>(p, grid, valu_rows, waves, s, ev_start, ev_stop);
  return hipErrorInvalidValue;
}


template <bool LAYERS>
hipError_t launch_direct_t(const AttnParams& p, dim3 grid, int32_t head_dim, int32_t stride, int32_t max_tok,
                           hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const uint4* kl = layer_head_base(p, p.k_pool, 0, head_dim);
  const uint4* vl = layer_head_base(p, p.v_pool, 0, head_dim);
  const uint32_t blk_chunks = static_cast<uint32_t>(p.Hkv * p.B * head_dim / 8);
  const uint32_t g_log2B = static_cast<uint32_t>(p.G) | (static_cast<uint32_t>(p.log2B) << 8);
  // eight waves at head_dim 64; at 128 a wave's loads in flight need more
  // registers than eight waves per workgroup leave, so four.  At 64, calls
  // of at most 3 steps per wave (768 keys) load everything in one round.
  constexpr int kAllSteps = 3;
  // With more workgroups than CUs, calls of at most kStepSlots steps keep
  // their V tiles in one step-indexed array that the merge area overlays
  // (74 KB of LDS instead of 133): two workgroups per CU, so one's loads
  // overlap the other's math and merge.  With fewer, the separate merge area
  // saves the barrier before the merge.
  constexpr int kStepSlots = 18;
  const int64_t n_wg = static_cast<int64_t>(grid.x) * grid.y * grid.z;
  if (head_dim == 64 && max_tok <= kStepSlots * kStep && n_wg > 256)
    hipExtLaunchKernelGGL((direct_kernel<64, 8, kAllSteps, true, LAYERS, kStepSlots>), grid, dim3(512), 0, s, ev_start,
                          ev_stop, 0, p.items, p.blocks, p.q, stride, p.Hq, g_log2B, blk_chunks, kl, vl, p);
  else if (head_dim == 64 && max_tok <= kAllSteps * 8 * kStep)
    hipExtLaunchKernelGGL((direct_kernel<64, 8, kAllSteps, true, LAYERS>), grid, dim3(512), 0, s, ev_start, ev_stop, 0,
                          p.items, p.blocks, p.q, stride, p.Hq, g_log2B, blk_chunks, kl, vl, p);
  else if (head_dim == 64)
    hipExtLaunchKernelGGL((direct_kernel<64, 8, 2, false, LAYERS>), grid, dim3(512), 0, s, ev_start, ev_stop, 0, p.items,
                          p.blocks, p.q, stride, p.Hq, g_log2B, blk_chunks, kl, vl, p);
  else if (head_dim == 128)
    hipExtLaunchKernelGGL((direct_kernel<128, 4, 2, false, LAYERS>), grid, dim3(256), 0, s, ev_start, ev_stop, 0,
                          p.items, p.blocks, p.q, stride, p.Hq, g_log2B, blk_chunks, kl, vl, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_direct(const AttnParams& p, int32_t n_items, int32_t head_dim, int32_t stride,
                         int32_t max_tok, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop, int32_t n_layers) {
  if (n_items == 0) return hipSuccess;
  if (stride < 1 || stride > kMaxItemBlocks || p.G > 16 || n_layers < 1 || n_layers > 65535)
    return hipErrorInvalidValue;
  const int64_t n_wg = static_cast<int64_t>(n_items) * p.Hkv * n_layers;
  if (n_wg > INT32_MAX) return hipErrorInvalidValue;
  if (n_items > 65535) return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>(p.Hkv), static_cast<uint32_t>(n_items), static_cast<uint32_t>(n_layers));
  return n_layers > 1 ? launch_direct_t<true>(p, grid, head_dim, stride, max_tok, s, ev_start, ev_stop)
                      : launch_direct_t<false>(p, grid, head_dim, stride, max_tok, s, ev_start, ev_stop);
}

}  // namespace pkv
