// Path items of a tree decode plan: a decode call over prefix-sharing
// branches -- a search tree's shared root, the levels below it, each leaf's
// own keys (SGLang RadixAttention page, measured benchmark: many branches
// over one parent; decode is bound by memory bandwidth, KV-cache lifecycle
// section).
//
// One workgroup of eight waves per (path item, kv head).  The item holds up
// to 32 rows (its queries x the G query heads of the kv head) as two 16-row
// MFMA tiles, and a list of 32-token steps, each from one segment of the
// trie and seen by the queries in its mask.  Wave w takes steps w, w + 8,
// ...; each wave has a K and a V tile of its own in LDS, filled by
// global_load_lds_dwordx4: the next step's K as soon as this step's score
// products have read the K tile, its V once the P V products have read the
// V tile.  The waves never wait for each other until the end.  Per step and
// tile: S^T = K Q^T (v_mfma_f32_16x16x32_bf16; A = K rows from LDS, shared
// by both tiles, B = the tile's Q in registers), the masked online softmax,
// and O^T += V^T P^T (V^T from the transposing LDS read), the row sums from
// the same product against a tile of ones.  At the end the eight waves'
// states and the queries' partial states from MFMA items (an earlier
// launch) are combined by log-sum-exp and written as out / lse.
//
// The workgroups of one kv head read the head's shared segments at the same
// time; with the kv heads' workgroups interleaved in launch order (eight kv
// heads: each XCD runs one head) the repeats are served by that XCD's L2.
#include <hip/hip_ext.h>
#include <math.h>

#include "../kernels.hpp"
#include "common.hpp"
#include "tile.hpp"

namespace pkv {
namespace {

constexpr int kPathWaves = 8;
constexpr int kPathThreads = 64 * kPathWaves;
constexpr int kPathTiles = kPathMaxRows / 16;
constexpr float kPathLoShare = 16.f;   // residual term while a weight exceeds sum / 16

// The item's query rows (32 rows x D bf16, laid out as a K tile).  A
// wave's K and V tiles (32 tokens x D bf16 each) hold exactly its final
// state (32 rows x D fp32), which it writes there after its last step.
// Then, per row: the weights of its 8 wave states and up to 8 partial
// states, the partial states' rows, and the row's query.
template <int D>
struct PathSmem {
  alignas(16) char q[kPathMaxRows * D * 2];
  alignas(16) char slot[kPathWaves][2][kStep * D * 2];   // [wave][K, V]: the wave's step, then its state
  alignas(16) float m[kPathMaxRows][kPathWaves];
  alignas(16) float l[kPathMaxRows][kPathWaves];
  alignas(16) float wt[kPathMaxRows][2 * kPathWaves];    // [row][wave states 0..7, partial states 8..15]
  alignas(16) int32_t part[kPathMaxRows][kPathMaxParts]; // the partial states' rows, -1 past the last
  int32_t qrow[kPathMaxRows];
};
static_assert(kPathMaxParts == kPathWaves, "one weight lane per wave state and per partial state");
static_assert(kPathMaxRows == kStep, "the query rows fill one K tile layout");
static_assert(2 * kStep * 2 == kPathMaxRows * 4, "a wave's state fills its two tiles");

// column c (a multiple of 4) of row r in a wave's state: 16-byte groups rotated
// by the row, so a wave's stores of 16 rows spread over the banks
__device__ __forceinline__ int fin_col(int r, int c) { return c ^ ((r & 7) << 2); }

template <int D>
__global__ __launch_bounds__(kPathThreads) void path_kernel(const PathItem* __restrict__ items,
                                                          const PathStep* __restrict__ steps,
                                                          AttnParams p) {
  constexpr int NK = D / 32;
  constexpr int ND = D / 16;
  constexpr int CPR = D / 8;
  constexpr int RUNS = kStep * CPR / 64;   // 1 KB runs per K (or V) tile
  constexpr int Q4 = D / 4;
  constexpr int NT = kPathTiles;
  __shared__ PathSmem<D> sm;

  // consecutive workgroups take the kv heads of one item
  const int h = static_cast<int>(blockIdx.x) % p.Hkv;
  const int item = static_cast<int>(blockIdx.x) / p.Hkv;
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

  // At the end each thread weighs one state of one row: row wr, state ws
  // (the wave states 0..7, the row's partial states 8..15).  The row's
  // query and merge row are read now, so that their latency passes under
  // the steps.
  const int wr = tid >> 4;
  const int ws = tid & 15;
  const bool wr_ok = wr < R;
  const int w_merge = wr_ok ? it.merge[wr / G] : -1;
  const int w_qrow = it.q_index[wr_ok ? wr / G : 0];
  const int w_hq = h * G + wr % G;

  // The item's query rows go to LDS first, one 1 KB run per wave (laid out
  // as a K tile: slot c = 64 u + lane holds row c / CPR, chunk
  // (c % CPR) ^ tile_swz(row)), ahead of the first step's K and V; rows
  // past the item's last are read from its first row and zeroed below.
  constexpr int Q_RUNS = kPathMaxRows * CPR / 64;
  if (wave < Q_RUNS) {
    const int c = wave * 64 + lane;
    const int r = c / CPR;
    const int ch = (c % CPR) ^ tile_swz<D>(r);
    const int qj = r < R ? r / G : 0;
    int qi = it.q_index[0];
#pragma unroll
    for (int t = 1; t < kPathMaxQ; ++t) qi = qj == t ? it.q_index[t] : qi;
    const uint16_t* qrow = p.q + (static_cast<size_t>(qi) * p.Hq + h * G + (r < R ? r % G : 0)) * D;
    lds_dma16(reinterpret_cast<const uint4*>(qrow) + ch, sm.q + wave * 1024);
  }

  const uint4* kb = layer_head_base(p, p.k_pool, h, D);
  const uint4* vb = layer_head_base(p, p.v_pool, h, D);
  const uint32_t blk_chunks = static_cast<uint32_t>(p.Hkv * p.B * D / 8);
  const int bmask = p.B - 1;
  const int mine = wave < n_steps ? (n_steps - 1 - wave) / kPathWaves + 1 : 0;   // this wave's steps

  // K (V) of a step into the wave's K (V) tile: run u fills chunk slot
  // c = 64 u + lane, row c / CPR, chunk (c % CPR) ^ tile_swz(row).  A full
  // step (32 tokens) reads each lane's chunk at a fixed byte offset from its
  // block's base (its slot within the block: the row, past the step's first
  // slot); run u reads the step's first block when u < CPR / 4 (rows 0..15)
  // and its second otherwise.  A shorter step re-reads its last token in
  // the rows past its count (masked below), so every run stays in written
  // slots of the pool.
  uint32_t lane_off[RUNS];
#pragma unroll
  for (int u = 0; u < RUNS; ++u) {
    const int c = u * 64 + lane;
    const int r = c / CPR;
    const int ch = (c % CPR) ^ tile_swz<D>(r);
    lane_off[u] = static_cast<uint32_t>(((p.B == 16 ? (r & 15) : r) * CPR + ch) * 16);
  }
  auto issue = [&](const PathStep& ps, int kv) __attribute__((always_inline)) {
    const int off = ps.meta & 0xFF;
    const int n_tok = (ps.meta >> 8) & 0xFF;
    char* dst = sm.slot[wave][kv];
    const uint4* src = kv ? vb : kb;
    if (n_tok == kStep) {
      const char* at_a = reinterpret_cast<const char*>(
          src + static_cast<uint64_t>(static_cast<uint32_t>(ps.blk_a)) * blk_chunks + off * CPR);
      const char* at_b = reinterpret_cast<const char*>(
          src + static_cast<uint64_t>(static_cast<uint32_t>(ps.blk_b)) * blk_chunks + off * CPR);
#pragma unroll
      for (int u = 0; u < RUNS; ++u) lds_dma16_at(u < CPR / 4 ? at_a : at_b, lane_off[u], dst + u * 1024);
    } else {
      const int last = n_tok - 1;
#pragma unroll
      for (int u = 0; u < RUNS; ++u) {
        const int c = u * 64 + lane;
        const int r = c / CPR;
        const int ch = (c % CPR) ^ tile_swz<D>(r);
        const int t = min(r, last);
        const int blk = t < 16 ? ps.blk_a : ps.blk_b;
        lds_dma16(src + chunk_index(blk, blk_chunks, ((off + t) & bmask) * CPR + ch), dst + u * 1024);
      }
    }
  };

  // The wave's steps in a rotated order (the item's index picks the first):
  // the workgroups of one kv head then read different keys of a shared run
  // at any moment, and read-mostly steps from the L2 mix with steps from
  // HBM.  Step descriptors are read one step ahead of their use; the first
  // step's K and V are requested before the query rows.
  const int rot = mine > 0 ? item % mine : 0;
  auto step_at = [&](int k) __attribute__((always_inline)) {
    const int kk = k + rot < mine ? k + rot : k + rot - mine;
    return steps[step0 + wave + kPathWaves * kk];
  };
  PathStep cur{}, nxt{};
  if (mine > 0) {
    cur = step_at(0);
    nxt = step_at(mine > 1 ? 1 : 0);
    issue(cur, 0);
    issue(cur, 1);
  }

  // tile j's row l16 is item row 16 j + l16: query (16 j + l16) / G, head
  // (16 j + l16) % G of this kv head; tile_q[j]: the queries with rows in
  // tile j (a step whose mask holds them all needs no per-row mask there)
  int my_q[NT];
  bool row_ok[NT];
  uint32_t tile_q[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int first = (16 * j) / G;
    const int last = min(16 * j + 15, R - 1) / G;
    const int nb = last - first + 1;
    tile_q[j] = 16 * j < R ? (nb >= 32 ? ~0u : (1u << nb) - 1u) << first : 0u;
  }
  // the query rows: this wave's run has landed once at most the first
  // step's K and V runs are in flight (issued after it); the barrier makes
  // every wave's run visible
  if (mine > 0)
    wait_vmcnt<2 * RUNS>();
  else
    wait_vmcnt<0>();
  lds_barrier();
  bf16x8 qf[NT][NK];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int r = 16 * j + l16;
    row_ok[j] = r < R;
    my_q[j] = row_ok[j] ? r / G : 0;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      qf[j][kk] = row_ok[j] ? *reinterpret_cast<const bf16x8*>(sm.q + tile_byte<D>(r, 4 * kk + g4))
                            : bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }

  float m_run[NT];
  f32x4 o[NT][ND + 1];   // o[j][ND]: row sums (P V against a tile of ones)
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    m_run[j] = -INFINITY;
#pragma unroll
    for (int dt = 0; dt <= ND; ++dt) o[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8 ones = {0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80};
  const char* kt = sm.slot[wave][0];
  const char* vt = sm.slot[wave][1];
  for (int k = 0; k < mine; ++k) {
    // step k's K has landed (its V, issued last, may still be in flight;
    // everything issued before it has landed too)
    wait_vmcnt<RUNS>();
    const int n_tok = (cur.meta >> 8) & 0xFF;
    f32x4 sacc[NT][2];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      sacc[j][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      sacc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + tile_byte<D>(16 * tt + l16, 4 * kk + g4));
#pragma unroll
        for (int j = 0; j < NT; ++j)
          sacc[j][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[j][kk], sacc[j][tt], 0, 0, 0);
      }
    // the K tile's reads are done: the next step's K goes into it now, while
    // this step's softmax and P V run
    if (k + 1 < mine) {
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS reads have returned
      issue(nxt, 0);
    }
    // per tile: each lane holds keys 16 tt + 4 g4 + i of its row l16.  A
    // row's reference max moves only when the row's max passes it by more
    // than kSlack (to that max): P <= 2^kSlack, the O rescale is rare.
    float pv[NT][8];
    float mx[NT], m_new[NT];
    bool grow = false;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      float sv[8];
      if (n_tok == kStep && (cur.qmask & tile_q[j]) == tile_q[j]) {
        // every key of the step, every row of the tile
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[e] = sacc[j][e >> 2][e & 3];
      } else {
        const bool vis_row = row_ok[j] && ((cur.qmask >> my_q[j]) & 1u);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tok = 16 * (e >> 2) + 4 * g4 + (e & 3);
          sv[e] = (vis_row && tok < n_tok) ? sacc[j][e >> 2][e & 3] : -INFINITY;
        }
      }
      float m = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) m = fmaxf(m, sv[e]);
      mx[j] = xor32_max(xor16_max(m)) * p.scale_log2;
      m_new[j] = mx[j] > m_run[j] + kSlack ? mx[j] : m_run[j];
      grow = grow || m_new[j] != m_run[j];
      const float m_use = (m_new[j] == -INFINITY) ? 0.f : m_new[j];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[j][e] = fast_exp2(fmaf(sv[e], p.scale_log2, -m_use));
      // the weights are taken here, before the rescale branch (the compiler
      // would otherwise sink them past it, away from the score products)
      asm volatile("" ::"v"(pv[j][0]), "v"(pv[j][1]), "v"(pv[j][2]), "v"(pv[j][3]), "v"(pv[j][4]),
                   "v"(pv[j][5]), "v"(pv[j][6]), "v"(pv[j][7]));
    }
    if (__ballot(grow)) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float alpha = (m_run[j] == -INFINITY) ? 0.f : fast_exp2(m_run[j] - m_new[j]);
#pragma unroll
        for (int dt = 0; dt <= ND; ++dt) o[j][dt] *= alpha;
        m_run[j] = m_new[j];
      }
    }
    bf16x8 pf[NT];
    uint32_t ph[NT][4];
    bool need_lo = false;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) ph[j][e >> 1] = pack_bf16x2(pv[j][e], pv[j][e + 1]);
      uint4 hv = make_uint4(ph[j][0], ph[j][1], ph[j][2], ph[j][3]);
      pf[j] = *reinterpret_cast<bf16x8*>(&hv);
      // the row's largest weight of this step against its sum over the steps before
      const float m_use = (m_run[j] == -INFINITY) ? 0.f : m_run[j];
      const float p_top = mx[j] == -INFINITY ? 0.f : fast_exp2(mx[j] - m_use);
      need_lo = need_lo || (row_ok[j] && p_top * kPathLoShare > o[j][ND][0]);
    }
    auto vop = [&](int dt) __attribute__((always_inline)) {
      const int r = 4 * g4 + (l16 >> 2);
      const int c = 2 * dt + ((l16 & 3) >> 1);
      const int off = (l16 & 1) * 8;
      const v4i16 vlo = lds_read_tr16(vt + tile_byte<D>(r, c) + off);
      const v4i16 vhi = lds_read_tr16(vt + tile_byte<D>(16 + r, c) + off);
      return bf16x8{vlo[0], vlo[1], vlo[2], vlo[3], vhi[0], vhi[1], vhi[2], vhi[3]};
    };
    // V has landed: only the next step's K (issued after the score
    // products) may still be in flight
    if (k + 1 < mine)
      wait_vmcnt<RUNS>();
    else
      wait_vmcnt<0>();
#pragma unroll
    for (int dt = 0; dt <= ND; ++dt) {
      const bf16x8 a = dt < ND ? vop(dt) : ones;
#pragma unroll
      for (int j = 0; j < NT; ++j) o[j][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[j], o[j][dt], 0, 0, 0);
    }
    if (__ballot(need_lo)) {
      bf16x8 pfl[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        uint32_t pl[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2)
          pl[e >> 1] = pack_bf16x2(pv[j][e] - __uint_as_float(ph[j][e >> 1] << 16),
                                   pv[j][e + 1] - __uint_as_float(ph[j][e >> 1] & 0xFFFF0000u));
        uint4 lv = make_uint4(pl[0], pl[1], pl[2], pl[3]);
        pfl[j] = *reinterpret_cast<bf16x8*>(&lv);
      }
#pragma unroll
      for (int dt = 0; dt <= ND; ++dt) {
        const bf16x8 a = dt < ND ? vop(dt) : ones;
#pragma unroll
        for (int j = 0; j < NT; ++j)
          o[j][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pfl[j], o[j][dt], 0, 0, 0);
      }
    }
    // likewise the V tile once the products have read it
    if (k + 1 < mine) {
      __builtin_amdgcn_s_waitcnt(0xC07F);
      issue(nxt, 1);
    }
    cur = nxt;
    nxt = step_at(k + 2 < mine ? k + 2 : 0);
  }
  wait_vmcnt<0>();

  // ---- the eight waves' states, then the queries' partial states ----
  // a weight lane of a partial state requests its row and lse now; they
  // arrive while the waves leave their states in LDS
  int w_part = -1;
  float w_lse = -INFINITY;
  if (ws >= kPathWaves && w_merge >= 0) {
    const MergeRow& mr = p.merges[w_merge];
    if (ws - kPathWaves < mr.n_parts) {
      w_part = mr.inl[ws - kPathWaves];
      w_lse = p.part_lse[static_cast<size_t>(w_part) + w_hq];
    }
  }
  // this wave's tiles are free: its loads have landed (above) and its LDS
  // reads have returned
  __builtin_amdgcn_s_waitcnt(0xC07F);
  // (as 16-byte units, so that every access is one 128-bit LDS operation)
  float4* fo = reinterpret_cast<float4*>(sm.slot[wave][0]);
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int r = 16 * j + l16;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
      fo[(r * D + fin_col(r, 16 * dt + 4 * g4)) >> 2] = make_float4(o[j][dt][0], o[j][dt][1], o[j][dt][2], o[j][dt][3]);
    if (g4 == 0) {
      sm.m[r][wave] = m_run[j];
      sm.l[r][wave] = o[j][ND][0];
    }
  }
  lds_barrier();
  // Per row, 16 lanes: the row's common max over its states (a wave state
  // counts once it has a key), each state's scale, the row's total weight,
  // and the states' normalised weights.  The row's first lane writes its
  // lse.
  {
    float v = w_lse;
    float lw = 1.f;
    if (ws < kPathWaves) {
      lw = sm.l[wr][ws];
      v = lw > 0.f ? sm.m[wr][ws] : -INFINITY;
    }
    const float mx = group_max<16>(v);
    const float e = v == -INFINITY ? 0.f : fast_exp2(v - mx);
    const float total = group_sum<16>(e * lw);
    sm.wt[wr][ws] = total > 0.f ? e / total : 0.f;
    if (ws >= kPathWaves) sm.part[wr][ws - kPathWaves] = w_part;
    if (ws == 0) {
      sm.qrow[wr] = w_qrow;
      if (wr_ok && p.lse) p.lse[static_cast<size_t>(w_qrow) * p.Hq + w_hq] = (mx + log2f(total)) * kLn2;
    }
  }
  lds_barrier();
  // Four consecutive dims of one row per thread and unit: the weighted sum
  // of the row's wave states and partial states.
  constexpr int NU = (kPathMaxRows * Q4 + kPathThreads - 1) / kPathThreads;
#pragma unroll
  for (int i = 0; i < NU; ++i) {
    const int u = tid + kPathThreads * i;
    if (u >= R * Q4) break;
    const int row = u / Q4;
    const int c = (u % Q4) * 4;
    const float4* wrow = reinterpret_cast<const float4*>(sm.wt[row]);
    const float4 wa = wrow[0];
    const float4 wb = wrow[1];
    const float wv[kPathWaves] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kPathWaves; ++w) {
      const float4 x = reinterpret_cast<const float4*>(sm.slot[w][0])[(row * D + fin_col(row, c)) >> 2];
      acc.x = fmaf(wv[w], x.x, acc.x);
      acc.y = fmaf(wv[w], x.y, acc.y);
      acc.z = fmaf(wv[w], x.z, acc.z);
      acc.w = fmaf(wv[w], x.w, acc.w);
    }
    const int hq = h * G + row % G;
    if (sm.part[row][0] >= 0) {
      const int4 ia = reinterpret_cast<const int4*>(sm.part[row])[0];
      const int4 ib = reinterpret_cast<const int4*>(sm.part[row])[1];
      const int pi[kPathMaxParts] = {ia.x, ia.y, ia.z, ia.w, ib.x, ib.y, ib.z, ib.w};
      const float4 pa = wrow[2];
      const float4 pb = wrow[3];
      const float pw[kPathMaxParts] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
      float4 y[kPathMaxParts];
#pragma unroll
      for (int k = 0; k < kPathMaxParts; ++k)
        y[k] = pi[k] >= 0 ? *reinterpret_cast<const float4*>(p.part_o + (static_cast<size_t>(pi[k]) + hq) * D + c)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int k = 0; k < kPathMaxParts; ++k) {
        acc.x = fmaf(pw[k], y[k].x, acc.x);
        acc.y = fmaf(pw[k], y[k].y, acc.y);
        acc.z = fmaf(pw[k], y[k].z, acc.z);
        acc.w = fmaf(pw[k], y[k].w, acc.w);
      }
    }
    const size_t orow = static_cast<size_t>(sm.qrow[row]) * p.Hq + hq;
    *reinterpret_cast<float4*>(p.out + orow * D + c) = acc;
  }
}

}  // namespace

hipError_t launch_path(const AttnParams& p, const PathItem* items, int32_t n_items, int32_t head_dim,
                       hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (n_items == 0) return hipSuccess;
  if (p.G > 16 || p.B < 16) return hipErrorInvalidValue;
  const int64_t n_wg = static_cast<int64_t>(n_items) * p.Hkv;
  if (n_wg > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>(n_wg));
  if (head_dim == 64)
    hipExtLaunchKernelGGL((path_kernel<64>), grid, dim3(kPathThreads), 0, s, ev_start, ev_stop, 0, items,
                          p.steps, p);
  else if (head_dim == 128)
    hipExtLaunchKernelGGL((path_kernel<128>), grid, dim3(kPathThreads), 0, s, ev_start, ev_stop, 0, items,
                          p.steps, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
