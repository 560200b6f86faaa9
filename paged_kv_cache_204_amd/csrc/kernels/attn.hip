// Paged attention over the block pool: one launch per call.
//
// Each workgroup (256 threads, blockIdx.y = kv head) runs one work item from
// the plan -- a run of key tokens reached through the block table and up to
// a tile of query rows (row groups x the G query heads of this kv head):
//
//  * MFMA items (blockIdx.x < n_mfma): the query tile is a real dense
//    contraction -- every node of a draft tree (CAST page, technical
//    summary "Problem": the target checks the whole tree in one pass) or a
//    shared prefix under many queries.  4 waves x RT row tiles of 16 rows.
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
#include <math.h>

#include "../kernels.hpp"
#include "common.hpp"

namespace pkv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kThreads = 256;

// K or V of layer p.layer, kv head h, as 16-byte chunks: token slot `off` of
// block `blk` starts at chunk blk * (Hkv * B * D / 8) + off * D / 8.  The pool
// creation keeps a layer under 2^32 chunks and a block under 2^24 chunks, so
// the index is one 24-bit multiply-add in 32 bits.
__device__ __forceinline__ const uint4* layer_head_base(const AttnParams& p, const uint16_t* pool,
                                                        int h, int D) {
  const size_t blk_stride = static_cast<size_t>(p.Hkv) * p.B * D;
  return reinterpret_cast<const uint4*>(pool + static_cast<size_t>(p.layer) * p.N * blk_stride +
                                        static_cast<size_t>(h) * p.B * D);
}

__device__ __forceinline__ uint32_t chunk_index(int32_t blk, uint32_t blk_chunks, int32_t within) {
  return __umul24(static_cast<uint32_t>(blk), blk_chunks) + static_cast<uint32_t>(within);
}

// ---------------------------------------------------------------- MFMA path
constexpr int kStep = 32;          // key tokens per step (two 16-token tiles)
constexpr int kDepth = 2;          // steps of K/V requested ahead
constexpr float kSlack = 8.f;      // log2 headroom of P above the reference max

template <int D>
struct MfmaSmem {
  uint16_t k[2][kStep][D + 8];     // K rows, padded pitch
  uint16_t vt[2][D][kStep + 4];    // V^T, pitch 18 words
};

// S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = K rows from LDS, B = Q rows
// in registers): the accumulator gives each lane 4 tokens of ONE query row,
// so the softmax max / sum need two cross-row swaps only, and the rounded P
// (bf16) of the lane's 8 tokens is exactly the B operand of O^T += V^T P^T.
// O^T keeps each lane on the same row, so the online rescale is lane local.
// The O rescale runs only when some row of the wave outgrows its reference
// max by more than kSlack (see the softmax step below).
template <int D, int RT>
__device__ __forceinline__ void mfma_item(const AttnParams& p, const WorkItem& it, int h,
                                          MfmaSmem<D>& sm, const int32_t* blk_s) {
  constexpr int NK = D / 32;
  constexpr int ND = D / 16;
  constexpr int CPR = D / 8;
  constexpr int KPER = kStep * CPR / kThreads;   // K chunks per thread per step
  constexpr int VUNITS = 16 * CPR;               // (token pair, chunk) units per step
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  // Staging: K chunk ci = tid + 256 i is (token ci / CPR, 16-byte chunk
  // ci % CPR); V unit tid is chunk (tid / 16) of tokens 2q and 2q + 1
  // (q = tid % 16), written transposed as 32-bit words (one dim, two tokens)
  // -- with the 18-word V^T pitch the 64 lanes of a store hit 64 banks.
  const bool v_on = tid < VUNITS;
  const int v_pair = tid & 15;
  const int v_c = (tid >> 4) % CPR;
  const uint4* kb = layer_head_base(p, p.k_pool, h, D);
  const uint4* vb = layer_head_base(p, p.v_pool, h, D);
  const uint32_t blk_chunks = static_cast<uint32_t>(p.Hkv * p.B * D / 8);
  const int t_last = it.n_tok - 1;
  auto ldg = [&](const uint4* src, int t, int c) {
    t = min(t, t_last);
    return src[chunk_index(blk_s[t >> p.log2B], blk_chunks, (t & (p.B - 1)) * (D / 8) + c)];
  };
  uint4 rk[kDepth][KPER], rv[kDepth][2];
  auto fetch = [&](int slot, int t0) {
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int ci = tid + kThreads * i;
      rk[slot][i] = ldg(kb, t0 + ci / CPR, ci % CPR);
    }
    rv[slot][0] = ldg(vb, t0 + 2 * v_pair, v_c);
    rv[slot][1] = ldg(vb, t0 + 2 * v_pair + 1, v_c);
  };
  const int nsteps = (it.n_tok + kStep - 1) / kStep;

  auto step = [&](int slot, int s) {
    const int buf = s & 1;
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int ci = tid + kThreads * i;
      *reinterpret_cast<uint4*>(&sm.k[buf][ci / CPR][(ci % CPR) * 8]) = rk[slot][i];
    }
    if (v_on) {
      const uint32_t a[4] = {rv[slot][0].x, rv[slot][0].y, rv[slot][0].z, rv[slot][0].w};
      const uint32_t b[4] = {rv[slot][1].x, rv[slot][1].y, rv[slot][1].z, rv[slot][1].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // (low halves of a and b), (high halves of a and b)
        *reinterpret_cast<uint32_t*>(&sm.vt[buf][v_c * 8 + 2 * j][2 * v_pair]) =
            __builtin_amdgcn_perm(b[j], a[j], 0x05040100u);
        *reinterpret_cast<uint32_t*>(&sm.vt[buf][v_c * 8 + 2 * j + 1][2 * v_pair]) =
            __builtin_amdgcn_perm(b[j], a[j], 0x07060302u);
      }
    }
    lds_barrier();
    fetch(slot, (s + kDepth) * kStep);
    if (!active) return;

    const int t0 = s * kStep;
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
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.k[buf][16 * tt + l16][32 * kk + 8 * g4]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          sacc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[rt][kk], sacc[rt][tt], 0, 0, 0);
      }
    }
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
      mx = xor32_max(xor16_max(mx)) * p.scale_log2;
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
        const float p0 = fast_exp2(fmaf(sv[j], p.scale_log2, -m_use));
        const float p1 = fast_exp2(fmaf(sv[j + 1], p.scale_log2, -m_use));
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
      const uint2 lo = *reinterpret_cast<const uint2*>(&sm.vt[buf][16 * dt + l16][4 * g4]);
      const uint2 hi = *reinterpret_cast<const uint2*>(&sm.vt[buf][16 * dt + l16][16 + 4 * g4]);
      uint4 av = make_uint4(lo.x, lo.y, hi.x, hi.y);
      const bf16x8 a = *reinterpret_cast<bf16x8*>(&av);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[rt], o[rt][dt], 0, 0, 0);
        o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf_lo[rt], o[rt][dt], 0, 0, 0);
      }
    }
  };

#pragma unroll
  for (int j = 0; j < kDepth; ++j) fetch(j, j * kStep);
  // whole rounds of the ring in the loop, the last partial round peeled, so
  // the loop body has no load behind a branch and the waits before each
  // staging store can count the loads still in flight
  int s0 = 0;
  for (; s0 + kDepth <= nsteps; s0 += kDepth) {
#pragma unroll
    for (int j = 0; j < kDepth; ++j) step(j, s0 + j);
  }
#pragma unroll
  for (int j = 0; j < kDepth - 1; ++j)
    if (s0 + j < nsteps) step(j, s0 + j);

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
constexpr int kValuRows = 8;     // query rows per item at most
constexpr int kValuTok = 512;    // key tokens per item
constexpr int kUnroll = 4;       // token passes with loads in flight per thread

template <int D>
struct alignas(16) ValuSmem {
  float s[kValuTok][kValuRows];   // scores, then probabilities, token-major
  float red[kThreads / 64][kValuRows][D];
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

// A token's head_dim row is read by D/8 lanes (128-bit loads, whole row
// coalesced); K and V of the first passes are requested together.  Phase 1
// forms the scores of every row for the item's keys (v_dot2_f32_bf16, a DPP
// butterfly over the row's lanes) into LDS, token-major; phase 2 takes an
// exact two-pass softmax per row (one wave per row); phase 3 accumulates
// p * v over each lane's tokens for its 8 dims (the 8 rows' p of a token are
// two 128-bit LDS reads) and sums lanes and waves holding the same dims.
// RM (4 or 8) bounds the rows at compile time; rows >= R compute on zero
// queries and are never written.
template <int D, int RM>
__device__ __forceinline__ void valu_item(const AttnParams& p, const WorkItem& it, int h,
                                          ValuSmem<D>& sm, const int32_t* blk_s) {
  constexpr int CPR = D / 8;
  constexpr int TPP = kThreads / CPR;
  static_assert(RM <= CPR, "one score row per lane of a token group");
  const int G = p.G;
  const int R = it.n_grp * G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = tid % CPR;
  const int tp = tid / CPR;

  const uint4* kb = layer_head_base(p, p.k_pool, h, D);
  const uint4* vb = layer_head_base(p, p.v_pool, h, D);
  const uint32_t blk_chunks = static_cast<uint32_t>(p.Hkv * p.B * D / 8);
  const int t_last = it.n_tok - 1;
  auto addr = [&](int t) {
    t = min(t, t_last);
    return chunk_index(blk_s[t >> p.log2B], blk_chunks, (t & (p.B - 1)) * (D / 8) + c);
  };
  const int npass = (it.n_tok + TPP - 1) / TPP;

  // first passes of K and V, then the queries
  uint4 kv[kUnroll], vv[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) kv[u] = kb[addr(u * TPP + tp)];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) vv[u] = vb[addr(u * TPP + tp)];
  uint4 qv[RM];
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    qv[r] = make_uint4(0, 0, 0, 0);
    if (r < R) {
      const RowGroup g = p.groups[it.grp_off + r / G];
      const size_t qoff = (static_cast<size_t>(g.q_index) * p.Hq + h * G + r % G) * D + c * 8;
      qv[r] = *reinterpret_cast<const uint4*>(p.q + qoff);
    }
  }
  uint64_t anc_mine = 0;
  if (c < R) {
    const RowGroup g = p.groups[it.grp_off + c / G];
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
  // ---- phase 2: exact softmax per row -----------------------------------------
  for (int r = wave; r < R; r += kThreads / 64) {
    float mx = -INFINITY;
    for (int t = lane; t < it.n_tok; t += 64) mx = fmaxf(mx, sm.s[t][r]);
    mx = wave_max(mx);
    const float m_use = (mx == -INFINITY) ? 0.f : mx;
    float sum = 0.f;
    for (int t = lane; t < it.n_tok; t += 64) {
      const float e = fast_exp2(sm.s[t][r] - m_use);
      sm.s[t][r] = e;
      sum += e;
    }
    sum = wave_sum(sum);
    if (lane == 0) {
      sm.m[r] = mx;
      sm.l[r] = sum;
    }
  }
  lds_barrier();
  // ---- phase 3: O = P V --------------------------------------------------------
  float o[RM][8];
#pragma unroll
  for (int r = 0; r < RM; ++r)
#pragma unroll
    for (int j = 0; j < 8; ++j) o[r][j] = 0.f;
  for (int p0 = 0; p0 < npass; p0 += kUnroll) {
    if (p0 > 0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) vv[u] = vb[addr((p0 + u) * TPP + tp)];
    }
    float pr[kUnroll][RM];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = (p0 + u) * TPP + tp;
      const int tc = min(t, t_last);
      const float4 a = *reinterpret_cast<const float4*>(&sm.s[tc][0]);
      pr[u][0] = a.x; pr[u][1] = a.y; pr[u][2] = a.z; pr[u][3] = a.w;
      if constexpr (RM == 8) {
        const float4 b = *reinterpret_cast<const float4*>(&sm.s[tc][4]);
        pr[u][4] = b.x; pr[u][5] = b.y; pr[u][6] = b.z; pr[u][7] = b.w;
      }
      if (t > t_last) {
#pragma unroll
        for (int r = 0; r < RM; ++r) pr[u][r] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float v[8] = {bf16_lo(vv[u].x), bf16_hi(vv[u].x), bf16_lo(vv[u].y), bf16_hi(vv[u].y),
                          bf16_lo(vv[u].z), bf16_hi(vv[u].z), bf16_lo(vv[u].w), bf16_hi(vv[u].w)};
#pragma unroll
      for (int r = 0; r < RM; ++r)
#pragma unroll
        for (int j = 0; j < 8; ++j) o[r][j] = fmaf(pr[u][r], v[j], o[r][j]);
    }
  }
  // lanes of a wave that hold the same dims (token slots tp) sum up ...
#pragma unroll
  for (int r = 0; r < RM; ++r) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float x = o[r][j];
      if constexpr (CPR == 8) x += dpp_f32<kDppXor8>(x);
      o[r][j] = xor32_sum(xor16_sum(x));
    }
  }
  // ... then the waves
  if (lane < CPR) {
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
    const float4 val = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    const RowGroup g = p.groups[it.grp_off + r / G];
    const int hq = h * G + r % G;
    if (it.part_base < 0) {
      const size_t row = static_cast<size_t>(g.q_index) * p.Hq + hq;
      *reinterpret_cast<float4*>(p.out + row * D + d) = val;
      if (p.lse && d == 0) p.lse[row] = (m + log2f(l)) * kLn2;
    } else {
      const size_t row = static_cast<size_t>(it.part_base) + static_cast<size_t>(r / G) * p.Hq + hq;
      *reinterpret_cast<float4*>(p.part_o + row * D + d) = val;
      if (d == 0) p.part_lse[row] = l > 0.f ? m + log2f(l) : -INFINITY;
    }
  }
}

template <int D, int RT, int RM>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnParams p) {
  __shared__ union alignas(16) {
    MfmaSmem<D> m;
    ValuSmem<D> v;
  } sm;
  __shared__ int32_t blk_s[kMaxItemBlocks];

  // the block list sits at a stride fixed per item kind, so its loads go
  // out together with the item's
  const bool is_mfma = static_cast<int>(blockIdx.x) < p.n_mfma;
  const int nb = is_mfma ? p.stride_mfma : p.stride_valu;
  const int32_t* lst = p.blocks + (is_mfma ? static_cast<size_t>(blockIdx.x) * p.stride_mfma
                                           : static_cast<size_t>(p.n_mfma) * p.stride_mfma +
                                                 static_cast<size_t>(blockIdx.x - p.n_mfma) * p.stride_valu);
  for (int i = threadIdx.x; i < nb; i += kThreads) blk_s[i] = lst[i];
  const WorkItem it = p.items[blockIdx.x];
  const int h = blockIdx.y;
  lds_barrier();
  if (static_cast<int>(blockIdx.x) < p.n_mfma)
    mfma_item<D, RT>(p, it, h, sm.m, blk_s);
  else
    valu_item<D, RM>(p, it, h, sm.v, blk_s);
}

}  // namespace

template <int D, int RT>
hipError_t launch_rows(const AttnParams& p, dim3 grid, int32_t valu_rows, hipStream_t s) {
  if (valu_rows <= 4)
    hipLaunchKernelGGL((attn_kernel<D, RT, 4>), grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((attn_kernel<D, RT, 8>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnParams& p, int32_t n_items, int32_t head_dim, int32_t row_tiles,
                       int32_t valu_rows, hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(n_items), static_cast<uint32_t>(p.Hkv));
  if (head_dim == 64 && row_tiles == 1) return launch_rows<64, 1>(p, grid, valu_rows, s);
  if (head_dim == 64 && row_tiles == 2) return launch_rows<64, 2>(p, grid, valu_rows, s);
  if (head_dim == 128 && row_tiles == 1) return launch_rows<128, 1>(p, grid, valu_rows, s);
  if (head_dim == 128 && row_tiles == 2) return launch_rows<128, 2>(p, grid, valu_rows, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv
