// 4-bit K/V: quantization on append and decode attention from the codes.
//
// The Dendrite page keeps the KV cache in 4 bits (TurboQuant) for 3.88x
// less memory and computes from the quantized indices rather than
// dequantizing the cache on every call.  Format of one head vector x of one
// token (head_dim D): its norm in fp16 and D 4-bit codes of the rotated
// direction H diag(s) x / (sqrt(D) |x|) -- H the Sylvester Hadamard matrix,
// s random signs given at pool creation -- each coordinate, times sqrt(D),
// quantized with the 16-level Lloyd-Max levels of the unit normal (J. Max,
// "Quantizing for minimum distortion", 1960).  2 + D/2 bytes per vector:
// 256 / 66 = 3.88 at D = 128.
//
// Quantize: one wave per vector, lane i holds dims 2i and 2i + 1.  The
// butterfly H (s * x) runs in float64 across lanes; for bf16 inputs every
// partial sum is exact, so the comparison of y^2 with b_k^2 * sum(x^2)
// (decision level b_k) is decided exactly, the same on any implementation.
//
// Decode: one workgroup per (query, kv head).  The G query rows are rotated
// once, qh = H (s * q); in the rotated space a key's score is
// (scale / D) * norm_k * sum_d qh_d level(code_d), so the MFMA contracts qh
// with the codes' levels (fp16, from a byte -> two-levels table) and never
// forms a dequantized key; V is accumulated in the rotated space, acc_d =
// sum_t p_t norm_t level(code_t,d), and rotated back once at the end:
// out = s * (H acc) / (D l).
#include <hip/hip_ext.h>
#include <hip/hip_fp16.h>

#include <algorithm>

#include "../kernels.hpp"
#include "common.hpp"

namespace pkv {
namespace {

// The norm is the fp16 value nearest to sqrt(sum x^2), ties to even.
//
// Max (1960), 16 levels, unit-variance Gaussian, ascending; decision levels
// of the positive half.
__constant__ float kLevels[16] = {-2.7326f, -2.0690f, -1.6180f, -1.2562f, -0.9423f, -0.6568f,
                                  -0.3881f, -0.1284f, 0.1284f,  0.3881f,  0.6568f,  0.9423f,
                                  1.2562f,  1.6180f,  2.0690f,  2.7326f};
constexpr double kDecision[7] = {0.2582, 0.5224, 0.7996, 1.0993, 1.4371, 1.8435, 2.4008};

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
  return __shfl_xor(v, m, 64);
}

// code of coordinate y of H (s * x), S = sum x^2: exact float64 decisions
__device__ __forceinline__ uint32_t q4_code(double y, double S) {
  const double y2 = __dmul_rn(y, y);
  uint32_t level = 0;
#pragma unroll
  for (int k = 0; k < 7; ++k) level += y2 > __dmul_rn(kDecision[k] * kDecision[k], S) ? 1u : 0u;
  return y >= 0.0 ? 8u + level : 7u - level;
}

__device__ __forceinline__ double half_value(uint32_t bits) {
  return static_cast<double>(__half2float(__ushort_as_half(static_cast<uint16_t>(bits))));
}

// fp16 nearest to sqrt(S), ties to even.  The fp32 route gives a candidate
// within one fp16 step; the squares of the fp16 midpoints around it (12
// significant bits, so exact in float64) are compared with S, which is
// exact too, and the candidate moves to the right neighbour if needed.
__device__ __forceinline__ uint16_t half_of_sqrt(double S) {
  uint32_t h = __half_as_ushort(__float2half_rn(static_cast<float>(sqrt(S))));
  if (h >= 0x7c00u) return 0x7c00u;   // beyond the fp16 range: +inf
  for (int it = 0; it < 2; ++it) {
    const double v = half_value(h);
    if (h > 0) {
      const double lo = 0.5 * (v + half_value(h - 1));
      const double lo2 = __dmul_rn(lo, lo);
      if (S < lo2 || (S == lo2 && (h & 1u))) {
        --h;
        continue;
      }
    }
    if (h < 0x7bffu) {
      const double hi = 0.5 * (v + half_value(h + 1));
      const double hi2 = __dmul_rn(hi, hi);
      if (S > hi2 || (S == hi2 && (h & 1u))) {
        ++h;
        continue;
      }
    }
    break;
  }
  return static_cast<uint16_t>(h);
}

__global__ __launch_bounds__(256) void q4_append_kernel(Q4AppendParams p) {
  const int D = p.D;
  const int half = D / 2;
  const int lane = threadIdx.x & 63;
  const int64_t n_vec = static_cast<int64_t>(p.L) * p.n_rows * p.Hkv * 2;
  const int64_t waves = static_cast<int64_t>(gridDim.x) * 4;
  for (int64_t v = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6); v < n_vec; v += waves) {
    int64_t r = v;
    const int kv = static_cast<int>(r & 1);
    r >>= 1;
    const int h = static_cast<int>(r % p.Hkv);
    r /= p.Hkv;
    const int row = static_cast<int>(r % p.n_rows);
    const int l = static_cast<int>(r / p.n_rows);
    const uint16_t* src = (kv ? p.v_new : p.k_new) +
                          ((static_cast<int64_t>(l) * p.n_rows + row) * p.Hkv + h) * D;
    const bool on = lane < half;
    double x0 = 0.0, x1 = 0.0;
    if (on) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(src + 2 * lane);
      x0 = static_cast<double>(bf16_lo(w));
      x1 = static_cast<double>(bf16_hi(w));
    }
    double S = __dadd_rn(__dmul_rn(x0, x0), __dmul_rn(x1, x1));
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) S = __dadd_rn(S, shfl_xor_f64(S, m));
    double y0 = 0.0, y1 = 0.0;
    if (on) {
      const double a = p.signs[2 * lane] * x0;
      const double b = p.signs[2 * lane + 1] * x1;
      y0 = a + b;
      y1 = a - b;
    }
    for (int m = 1; m < half; m <<= 1) {
      const double p0 = shfl_xor_f64(y0, m);
      const double p1 = shfl_xor_f64(y1, m);
      if (lane & m) {
        y0 = p0 - y0;
        y1 = p1 - y1;
      } else {
        y0 = y0 + p0;
        y1 = y1 + p1;
      }
    }
    const int32_t slot = p.slots[row];
    const int32_t blk = slot >> p.log2B;
    const int32_t off = slot & (p.B - 1);
    const int64_t vec = ((static_cast<int64_t>(l) * p.N + blk) * p.Hkv + h) * p.B + off;
    if (on) {
      const uint32_t c = q4_code(y0, S) | (q4_code(y1, S) << 4);
      (kv ? p.v_codes : p.k_codes)[vec * half + lane] = static_cast<uint8_t>(c);
    }
    if (lane == 0) (kv ? p.v_norms : p.k_norms)[vec] = half_of_sqrt(S);
  }
  // copy-on-write: the filled slots of shared blocks (codes and norms)
  const int64_t n_copy = static_cast<int64_t>(p.n_cow) * p.L * 2 * p.Hkv * p.B;
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; u < n_copy;
       u += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    int64_t r = u;
    const int slot = static_cast<int>(r % p.B);
    r /= p.B;
    const int h = static_cast<int>(r % p.Hkv);
    r /= p.Hkv;
    const int kv = static_cast<int>(r & 1);
    r >>= 1;
    const int l = static_cast<int>(r % p.L);
    const int ci = static_cast<int>(r / p.L);
    const int32_t src_blk = p.cow[3 * ci + 0];
    const int32_t dst_blk = p.cow[3 * ci + 1];
    if (slot >= p.cow[3 * ci + 2]) continue;
    const int64_t vs = ((static_cast<int64_t>(l) * p.N + src_blk) * p.Hkv + h) * p.B + slot;
    const int64_t vd = ((static_cast<int64_t>(l) * p.N + dst_blk) * p.Hkv + h) * p.B + slot;
    uint8_t* codes = kv ? p.v_codes : p.k_codes;
    uint16_t* norms = kv ? p.v_norms : p.k_norms;
    const uint4* s4 = reinterpret_cast<const uint4*>(codes + vs * half);
    uint4* d4 = reinterpret_cast<uint4*>(codes + vd * half);
    for (int i = 0; i < half / 16; ++i) d4[i] = s4[i];
    norms[vd] = norms[vs];
  }
}

// In-wave butterfly of one row of D floats, lane i holding dims 2i, 2i + 1.
__device__ __forceinline__ void fwht_f32(float& y0, float& y1, int lane, int half) {
  const float a = y0, b = y1;
  y0 = a + b;
  y1 = a - b;
  for (int m = 1; m < half; m <<= 1) {
    const float p0 = __shfl_xor(y0, m, 64);
    const float p1 = __shfl_xor(y1, m, 64);
    if (lane & m) {
      y0 = p0 - y0;
      y1 = p1 - y1;
    } else {
      y0 = y0 + p0;
      y1 = y1 + p1;
    }
  }
}

// ---- MFMA decode ------------------------------------------------------------
// One workgroup per (query, kv head) with W waves taking the 32-key steps in
// turn, as the bf16 direct decode does, but the MFMA operands come from the
// codes: a 256-entry LDS table turns each code byte into its two fp16
// levels, so 8 dims of a key are four table reads.  In the rotated space a
// key's score is (scale / D) * n_k * sum_d qh_d level_d, qh = H (s * q): the
// MFMA contracts qh (fp16) with the levels and the key norm scales the
// result; the V norm scales the probability before P.V.  A wave requests its
// next step's codes and norms before it computes the current one (two
// register sets in turn), and its first step's before the query rotation;
// the running output is rescaled only in steps that raise a row's max.  The
// waves' softmax states meet in LDS, and the merged rows are rotated back
// once.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef short v4i16q __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16q* lds_v4i16q_ptr;

constexpr int kQStep = 32;   // keys per step

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

__device__ __forceinline__ uint16_t f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

template <int D, int W>
union Q4Smem {
  uint16_t v[W][kQStep][D + 8];   // each wave's V tile as fp16 levels, padded pitch
  struct {
    float o[W][16][D + 4];
    float m[W][16];
    float l[W][16];
  } fin;
};

// K/V codes and norms of one 32-key step, as loaded: the next step's are
// requested before the current step is computed.
template <int D>
struct Q4StepRaw {
  uint32_t kw[2][D / 32];             // K operands: keys 16 tt + l16, dims 32 kk + 8 g4 ..
  uint32_t vw[kQStep * (D / 8) / 64]; // V chunks ci = lane + 64 i: key ci / CPR, chunk ci % CPR
  uint2 kn[2], vn[2];                 // norms: keys 16 tt + 4 g4 .. + 3 (blocks of 16 or more),
                                      // else key 16 tt + l16 in the low half of .x
};

template <int D, int W, bool BIG>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(D == 64 ? 4 : 2))) void q4_mfma_kernel(
    Q4DecodeParams p) {
  constexpr int NK = D / 32;
  constexpr int ND = D / 16;
  constexpr int CPR = D / 8;                 // 8-dim chunks per key row
  constexpr int VPER = kQStep * CPR / 64;    // V chunks per lane per step
  constexpr int HALF = D / 2;
  constexpr int RPW = 16 / W;                // rows of the 16-row query tile per wave
  __shared__ uint32_t pair_lut[256];         // code byte -> (fp16 level lo, hi)
  __shared__ __align__(16) float qrot[16][D];   // rotated query rows, then merged outputs
  __shared__ __align__(16) Q4Smem<D, W> sm;

  const int G = p.G;
  const int item = static_cast<int>(blockIdx.x) / p.Hkv;
  const int h = static_cast<int>(blockIdx.x) - item * p.Hkv;
  const Q4Item it = p.items[item];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(it.q_index) * p.Hq + static_cast<int64_t>(h) * G;

  const int64_t head_vecs = static_cast<int64_t>(p.Hkv) * p.B;
  const int64_t layer_vecs = head_vecs * p.N;
  const uint32_t* kc32 = reinterpret_cast<const uint32_t*>(p.k_codes);
  const uint32_t* vc32 = reinterpret_cast<const uint32_t*>(p.v_codes);
  const int t_last = it.n_tok - 1;
  auto vec_of = [&](int t) {
    t = min(t, t_last);
    const int32_t blk = p.blocks[it.blk_off + (t >> p.log2B)];
    return p.layer * layer_vecs + blk * head_vecs + static_cast<int64_t>(h) * p.B + (t & (p.B - 1));
  };
  // step s's codes and norms into d; keys past the end re-read the last key
  // (masked when the scores are formed)
  auto load_step = [&](int s, Q4StepRaw<D>& d) __attribute__((always_inline)) {
    const int t0 = s * kQStep;
    if constexpr (BIG) {
      // Each 16-key half of the step lies in one block (blocks of 16: the
      // step's first and second block; larger: one block), so a load takes
      // the half's block base, the same for the whole wave, and a 32-bit
      // lane offset.
      const int r_last = t_last - t0;
      const int32_t* tbl = p.blocks + it.blk_off;
      const int64_t va = p.layer * layer_vecs + static_cast<int64_t>(tbl[t0 >> p.log2B]) * head_vecs +
                         static_cast<int64_t>(h) * p.B + (t0 & (p.B - 1));
      const bool two = p.B == 16 && r_last >= 16;
      const int64_t vb = two ? p.layer * layer_vecs + static_cast<int64_t>(tbl[(t0 + 16) >> p.log2B]) * head_vecs +
                                   static_cast<int64_t>(h) * p.B
                             : va;
      const int off_b = two ? 16 : 0;   // key of the second half's base
      const uint32_t* kh[2] = {kc32 + va * (D / 8), kc32 + vb * (D / 8)};
      const uint32_t* vh[2] = {vc32 + va * (D / 8), vc32 + vb * (D / 8)};
      const uint16_t* knh[2] = {p.k_norms + va, p.k_norms + vb};
      const uint16_t* vnh[2] = {p.v_norms + va, p.v_norms + vb};
      const int hoff[2] = {0, off_b};
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const uint32_t r = static_cast<uint32_t>(min(16 * tt + l16, r_last) - hoff[tt]);
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) d.kw[tt][kk] = kh[tt][r * (D / 8) + 4 * kk + g4];
        // four consecutive keys' norms, one 8-byte load each (a group past
        // the end re-reads the half's last whole group, which may run past
        // the last key into unwritten slots: masked when the step is computed)
        const uint32_t r0 = static_cast<uint32_t>(min(16 * tt + 4 * g4, r_last & ~3) - hoff[tt]);
        d.kn[tt] = *reinterpret_cast<const uint2*>(knh[tt] + r0);
        d.vn[tt] = *reinterpret_cast<const uint2*>(vnh[tt] + r0);
      }
#pragma unroll
      for (int i = 0; i < VPER; ++i) {
        const int ci = lane + 64 * i;
        constexpr int KPI = 64 / CPR;               // keys per i: all in one half
        const int half = (KPI * i) >> 4;
        const uint32_t r = static_cast<uint32_t>(min(ci / CPR, r_last) - hoff[half]);
        d.vw[i] = vh[half][r * (D / 8) + ci % CPR];
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int64_t vec = vec_of(t0 + 16 * tt + l16);
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) d.kw[tt][kk] = kc32[vec * (D / 8) + 4 * kk + g4];
        d.kn[tt] = make_uint2(p.k_norms[vec], 0u);
        d.vn[tt] = make_uint2(p.v_norms[vec], 0u);
      }
#pragma unroll
      for (int i = 0; i < VPER; ++i) {
        const int ci = lane + 64 * i;
        d.vw[i] = vc32[vec_of(t0 + ci / CPR) * (D / 8) + ci % CPR];
      }
    }
  };
  auto h2f = [](uint32_t bits) { return __half2float(__ushort_as_half(static_cast<uint16_t>(bits))); };

  for (int i = tid; i < 256; i += 64 * W)
    pair_lut[i] = static_cast<uint32_t>(f16_bits(kLevels[i & 15])) |
                  (static_cast<uint32_t>(f16_bits(kLevels[i >> 4])) << 16);
  // The wave's query rows and signs are requested next, then its first
  // step's codes, so that their latency passes under the rotation.
  uint32_t qw[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int g = wave + W * i;
    qw[i] = (g < G && lane < HALF) ? *reinterpret_cast<const uint32_t*>(p.q + (row0 + g) * D + 2 * lane) : 0u;
  }
  const float2 sg = lane < HALF ? *reinterpret_cast<const float2*>(p.signs + 2 * lane) : make_float2(0.f, 0.f);
  // every query has a key (empty sequences are refused), so every wave
  // loads a step; a wave without steps of its own loads the last one and
  // leaves it unused
  const int nsteps = (it.n_tok + kQStep - 1) / kQStep;
  Q4StepRaw<D> cur, nxt;
  load_step(min(wave, nsteps - 1), cur);
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int g = wave + W * i;
    if (g >= G) {
      // rows of the tile past the group: zero operands, no rotation
      if (lane < HALF) {
        qrot[g][2 * lane] = 0.f;
        qrot[g][2 * lane + 1] = 0.f;
      }
      continue;
    }
    float y0 = sg.x * bf16_lo(qw[i]);
    float y1 = sg.y * bf16_hi(qw[i]);
    fwht_f32(y0, y1, lane, HALF);
    if (lane < HALF) {
      qrot[g][2 * lane] = y0;
      qrot[g][2 * lane + 1] = y1;
    }
  }
  // LDS only: the first step's loads stay in flight across the barrier
  lds_barrier();
  // B operand: row l16, dims 32 kk + 8 g4 .. + 7
  f16x8 qf[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[kk][e] = static_cast<_Float16>(qrot[l16][32 * kk + 8 * g4 + e]);

  auto levels8 = [&](uint32_t word) {
    const uint32_t a = pair_lut[word & 255u], b = pair_lut[(word >> 8) & 255u];
    const uint32_t c = pair_lut[(word >> 16) & 255u], d = pair_lut[word >> 24];
    const uint4 u = make_uint4(a, b, c, d);
    return __builtin_bit_cast(f16x8, u);
  };
  const float zscale = p.scale_log2 / static_cast<float>(D);
  float m_run = -INFINITY, l_run = 0.f;
  f32x4v o[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) o[dt] = f32x4v{0.f, 0.f, 0.f, 0.f};
  uint16_t (*vs)[D + 8] = sm.v[wave];

  // One step from its loaded codes and norms.
  auto compute_step = [&](int s, const Q4StepRaw<D>& cur) __attribute__((always_inline)) {
    const int t0 = s * kQStep;
    // norms of the keys this lane's scores hold (16 tt + 4 g4 + i)
    float knk[8], vnk[8];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if constexpr (BIG) {
        knk[4 * tt + 0] = h2f(cur.kn[tt].x);
        knk[4 * tt + 1] = h2f(cur.kn[tt].x >> 16);
        knk[4 * tt + 2] = h2f(cur.kn[tt].y);
        knk[4 * tt + 3] = h2f(cur.kn[tt].y >> 16);
        vnk[4 * tt + 0] = h2f(cur.vn[tt].x);
        vnk[4 * tt + 1] = h2f(cur.vn[tt].x >> 16);
        vnk[4 * tt + 2] = h2f(cur.vn[tt].y);
        vnk[4 * tt + 3] = h2f(cur.vn[tt].y >> 16);
      } else {
        const float kn_l = h2f(cur.kn[tt].x), vn_l = h2f(cur.vn[tt].x);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int src = 4 * g4 + i;                 // the lane that loaded key 16 tt + 4 g4 + i
          knk[4 * tt + i] = __shfl(kn_l, src, 64);
          vnk[4 * tt + i] = __shfl(vn_l, src, 64);
        }
      }
    }
    // V tile as fp16 levels (this wave's earlier reads of it are done)
    wave_sync_lds();
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int ci = lane + 64 * i;
      *reinterpret_cast<f16x8*>(&vs[ci / CPR][(ci % CPR) * 8]) = levels8(cur.vw[i]);
    }
    // S^T = K Q^T: lane (l16, g4) gets keys 16 tt + 4 g4 + i of row l16
    f32x4v sacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sacc[tt] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        sacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(levels8(cur.kw[tt][kk]), qf[kk], sacc[tt], 0, 0, 0);
    }
    // y = n_k * (qh . level): the logit before the factor zscale, which the
    // exponent applies (zscale > 0, so the max commutes with it)
    float y[8];
    if (t0 + kQStep <= it.n_tok) {
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = sacc[e >> 2][e & 3] * knk[e];
    } else {
      // keys past the end: no score, and no V norm (a norm group that runs
      // past the last key holds slots never written, whose bits may be inf
      // or NaN, and 0 * inf would reach P V)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = t0 + 16 * (e >> 2) + 4 * g4 + (e & 3);
        y[e] = tok < it.n_tok ? sacc[e >> 2][e & 3] * knk[e] : -INFINITY;
        vnk[e] = tok < it.n_tok ? vnk[e] : 0.f;
      }
    }
    float mx = y[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, y[j]);
    mx = xor32_max(xor16_max(mx)) * zscale;
    // the running max moves only when this step passes it; o and l are
    // rescaled then (they are still zero before the first step)
    const bool grow = mx > m_run;
    if (__ballot(grow && m_run != -INFINITY)) {
      const float alpha = (m_run == -INFINITY || !grow) ? 1.f : fast_exp2(m_run - mx);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) o[dt] *= alpha;
    }
    m_run = grow ? mx : m_run;                     // finite: every step holds a key
    f16x8 pf;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float pr = fast_exp2(fmaf(y[j], zscale, -m_run));
      l_run += pr;
      pf[j] = static_cast<_Float16>(pr * vnk[j]);
    }
    wave_sync_lds();
    // O^T += V^T P^T, V^T read transposed from the wave's tile
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      const int r = 4 * g4 + (l16 >> 2);
      const int c = 16 * dt + 4 * (l16 & 3);
      const v4i16q lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16q_ptr)(&vs[r][c]));
      const v4i16q hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16q_ptr)(&vs[16 + r][c]));
      const v4i16q both[2] = {lo, hi};
      const f16x8 a = __builtin_bit_cast(f16x8, both);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pf, o[dt], 0, 0, 0);
    }
  };
  // Two buffers in turn: the wave's next step is requested before the
  // current one is computed.  Each branch computes its own copy of the step,
  // so that the load-counter wait before it is fixed: the copy after a
  // request waits only for the older loads.
  if (wave < nsteps) {
    for (int s = wave;; s += 2 * W) {
      if (s + W < nsteps) {
        load_step(s + W, nxt);
        compute_step(s, cur);
      } else {
        compute_step(s, cur);
        break;
      }
      if (s + 2 * W < nsteps) {
        load_step(s + 2 * W, cur);
        compute_step(s + W, nxt);
      } else {
        compute_step(s + W, nxt);
        break;
      }
    }
  }
  // ---- merge of the W wave states, rotation back --------------------------
  const float l_w = xor32_sum(xor16_sum(l_run));
  __syncthreads();   // every wave is done with its V tile (aliased below)
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
    *reinterpret_cast<float4*>(&sm.fin.o[wave][l16][16 * dt + 4 * g4]) =
        make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
  if (g4 == 0) {
    sm.fin.m[wave][l16] = m_run;
    sm.fin.l[wave][l16] = l_w;
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += 64 * W) {
    const int row = e / D;
    const int d = e - row * D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) mx = fmaxf(mx, sm.fin.m[w][row]);
    float l = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = sm.fin.m[w][row];
      const float a = mw == -INFINITY ? 0.f : fast_exp2(mw - mx);
      l = fmaf(a, sm.fin.l[w][row], l);
      acc = fmaf(a, sm.fin.o[w][row][d], acc);
    }
    qrot[row][d] = acc / (static_cast<float>(D) * l);
    if (d == 0 && p.lse) p.lse[row0 + row] = (mx + log2f(l)) * kLn2;
  }
  __syncthreads();
  for (int g = wave; g < G; g += W) {
    float y0 = 0.f, y1 = 0.f;
    if (lane < HALF) {
      y0 = qrot[g][2 * lane];
      y1 = qrot[g][2 * lane + 1];
    }
    fwht_f32(y0, y1, lane, HALF);
    if (lane < HALF)
      *reinterpret_cast<float2*>(p.out + (row0 + g) * D + 2 * lane) =
          make_float2(p.signs[2 * lane] * y0, p.signs[2 * lane + 1] * y1);
  }
}

}  // namespace

hipError_t launch_q4_append(const Q4AppendParams& p, hipStream_t s) {
  const int64_t n_vec = static_cast<int64_t>(p.L) * p.n_rows * p.Hkv * 2;
  const int64_t n_copy = static_cast<int64_t>(p.n_cow) * p.L * 2 * p.Hkv * p.B;
  if (n_vec == 0 && n_copy == 0) return hipSuccess;
  int64_t blocks = std::max((n_vec + 3) / 4, (n_copy + 255) / 256);
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(q4_append_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_q4_decode(const Q4DecodeParams& p, int32_t n_items, int32_t head_dim,
                            hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (n_items == 0) return hipSuccess;
  const int64_t n_wg = static_cast<int64_t>(n_items) * p.Hkv;
  const dim3 grid(static_cast<uint32_t>(n_wg));
  // Waves per (query, kv head): the fewest that still occupy half of the
  // waves the GPU holds at once (four per SIMD at head_dim 64, two at 128),
  // since each added wave repeats the per-item set-up and merge; measured at
  // the Trellis shape, 1024 .. 4096 sessions run 25-30 % faster on one or two
  // waves than on eight, 16 .. 64 sessions faster on eight.  Blocks under 16
  // tokens keep the widest form.
  const int64_t target = head_dim == 64 ? 8 * 256 : 4 * 256;
  const int wmax = head_dim == 64 ? 8 : 4;
  int w = 1;
  while (w < wmax && n_wg * w < target) w *= 2;
  if (p.B < 16) w = wmax;
  auto go = [&](auto kernel, int threads) {
    hipExtLaunchKernelGGL(kernel, grid, dim3(threads), 0, s, ev_start, ev_stop, 0, p);
    return hipGetLastError();
  };
  if (head_dim == 64) {
    if (p.B < 16) return go(q4_mfma_kernel<64, 8, false>, 512);
    if (w == 1) return go(q4_mfma_kernel<64, 1, true>, 64);
    if (w == 2) return go(q4_mfma_kernel<64, 2, true>, 128);
    if (w == 4) return go(q4_mfma_kernel<64, 4, true>, 256);
    return go(q4_mfma_kernel<64, 8, true>, 512);
  }
  if (head_dim == 128) {
    if (p.B < 16) return go(q4_mfma_kernel<128, 4, false>, 256);
    if (w == 1) return go(q4_mfma_kernel<128, 1, true>, 64);
    if (w == 2) return go(q4_mfma_kernel<128, 2, true>, 128);
    return go(q4_mfma_kernel<128, 4, true>, 256);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
