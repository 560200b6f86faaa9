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
// once, qh = H (s * q), and turned into per-row tables T[d][c] = qh_d *
// level_c * scale / D (all rows of an entry side by side), so a key's score
// is norm * sum_d T[d][code_d] -- table
// lookups on the codes, no dequantized keys.  Chunks of 256 keys, one per
// thread, with an online softmax across chunks; V is accumulated in the
// rotated space, acc_d = sum_t p_t norm_t level(code_t,d), by lanes over
// dims, and rotated back once at the end: out = s * (H acc) / (D l).
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

constexpr int kChunk = 256;     // keys per chunk = threads per decode workgroup

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

template <int D>
__global__ __launch_bounds__(kChunk) void q4_decode_kernel(Q4DecodeParams p) {
  constexpr int HALF = D / 2;
  constexpr int MAXG = kQ4MaxRowDims / D;
  __shared__ __align__(16) float lut[kQ4MaxRowDims * 16];   // [d][code][g], MAXG rows
  __shared__ __align__(16) float sc[kChunk][MAXG];   // [key][row]: scores, then probabilities
  __shared__ __align__(16) uint8_t vcs[kChunk][HALF];   // V codes of the chunk
  __shared__ float accs[4][kQ4MaxRowDims];         // per-wave partial V sums [g][d]
  __shared__ float vn_s[kChunk];                   // V norms of the chunk
  __shared__ float m_s[MAXG], l_s[MAXG], a_s[MAXG];
  __shared__ float lv_s[16];

  const int G = p.G;
  const int item = static_cast<int>(blockIdx.x) / p.Hkv;
  const int h = static_cast<int>(blockIdx.x) - item * p.Hkv;
  const Q4Item it = p.items[item];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool on = lane < HALF;
  const int64_t row0 = static_cast<int64_t>(it.q_index) * p.Hq + static_cast<int64_t>(h) * G;
  if (tid < 16) lv_s[tid] = kLevels[tid];

  // rotated query rows -> lookup tables (scale, log2 e and 1/D folded in)
  const float tscale = p.scale_log2 / static_cast<float>(D);
  for (int g = wave; g < G; g += 4) {
    float y0 = 0.f, y1 = 0.f;
    if (on) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(p.q + (row0 + g) * D + 2 * lane);
      y0 = p.signs[2 * lane] * bf16_lo(w);
      y1 = p.signs[2 * lane + 1] * bf16_hi(w);
    }
    fwht_f32(y0, y1, lane, HALF);
    if (on) {
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        lut[((2 * lane) * 16 + c) * MAXG + g] = y0 * kLevels[c] * tscale;
        lut[((2 * lane + 1) * 16 + c) * MAXG + g] = y1 * kLevels[c] * tscale;
      }
    }
  }
  if (tid < MAXG) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }
  float acc0[MAXG], acc1[MAXG];
#pragma unroll
  for (int g = 0; g < MAXG; ++g) acc0[g] = acc1[g] = 0.f;
  __syncthreads();

  const int64_t head_vecs = static_cast<int64_t>(p.Hkv) * p.B;   // vectors per block and layer
  const int64_t layer_vecs = head_vecs * p.N;
  for (int c0 = 0; c0 < it.n_tok; c0 += kChunk) {
    const int t = c0 + tid;
    const int nt = min(kChunk, it.n_tok - c0);
    if (t < it.n_tok) {
      const int32_t blk = p.blocks[it.blk_off + (t >> p.log2B)];
      const int64_t vec = p.layer * layer_vecs + blk * head_vecs + static_cast<int64_t>(h) * p.B +
                          (t & (p.B - 1));
      const uint4* kc = reinterpret_cast<const uint4*>(p.k_codes + vec * HALF);
      const uint4* vc = reinterpret_cast<const uint4*>(p.v_codes + vec * HALF);
      uint32_t kw[HALF / 4];
#pragma unroll
      for (int i = 0; i < HALF / 16; ++i) {
        const uint4 a = kc[i];
        kw[4 * i + 0] = a.x;
        kw[4 * i + 1] = a.y;
        kw[4 * i + 2] = a.z;
        kw[4 * i + 3] = a.w;
        reinterpret_cast<uint4*>(vcs[tid])[i] = vc[i];
      }
      const float kn = __half2float(__ushort_as_half(p.k_norms[vec]));
      vn_s[tid] = __half2float(__ushort_as_half(p.v_norms[vec]));
      // one accumulator per row; the MAXG row values of a (dim, code) entry
      // are contiguous, so a key dim costs MAXG / 4 128-bit reads (rows past
      // G hold no data and are never used)
      float sg[MAXG];
#pragma unroll
      for (int g = 0; g < MAXG; ++g) sg[g] = 0.f;
#pragma unroll
      for (int w = 0; w < HALF / 4; ++w) {
        const uint32_t word = kw[w];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float4* e = reinterpret_cast<const float4*>(
              lut + ((8 * w + j) * 16 + ((word >> (4 * j)) & 15u)) * MAXG);
#pragma unroll
          for (int g4 = 0; g4 < MAXG / 4; ++g4) {
            const float4 v = e[g4];
            sg[4 * g4 + 0] += v.x;
            sg[4 * g4 + 1] += v.y;
            sg[4 * g4 + 2] += v.z;
            sg[4 * g4 + 3] += v.w;
          }
        }
      }
#pragma unroll
      for (int g = 0; g < MAXG; ++g) sc[tid][g] = sg[g] * kn;
    }
    __syncthreads();
    // per row: chunk max, new running max, probabilities (times the V norm)
    for (int g = wave; g < G; g += 4) {
      float mx = -INFINITY;
      for (int i = lane; i < nt; i += 64) mx = fmaxf(mx, sc[i][g]);
      mx = wave_max(mx);
      const float m_old = m_s[g];
      const float m_new = fmaxf(m_old, mx);
      const float alpha = m_old == -INFINITY ? 0.f : fast_exp2(m_old - m_new);
      float ps = 0.f;
      for (int i = lane; i < nt; i += 64) {
        const float pr = fast_exp2(sc[i][g] - m_new);
        ps += pr;
        sc[i][g] = pr;
      }
      ps = wave_sum(ps);
      if (lane == 0) {
        m_s[g] = m_new;
        l_s[g] = l_s[g] * alpha + ps;
        a_s[g] = alpha;
      }
    }
    __syncthreads();
    // V: lanes over dims (two per lane), waves over keys of the chunk
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {
      const float al = g < G ? a_s[g] : 0.f;
      acc0[g] *= al;
      acc1[g] *= al;
    }
    if (on) {
      // four keys per step, every load of the step issued before the sums;
      // keys past the chunk's end re-read its last key with weight 0
      for (int i0 = wave; i0 < nt; i0 += 16) {
        float l0[4], l1[4];
        int ic[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + 4 * u;
          ic[u] = min(i, nt - 1);
          const uint32_t byte = vcs[ic[u]][lane];
          const float vn = i < nt ? vn_s[ic[u]] : 0.f;
          l0[u] = lv_s[byte & 15u] * vn;
          l1[u] = lv_s[byte >> 4] * vn;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float4* pr4 = reinterpret_cast<const float4*>(sc[ic[u]]);
#pragma unroll
          for (int g4 = 0; g4 < MAXG / 4; ++g4) {
            const float4 pr = pr4[g4];
            acc0[4 * g4 + 0] = fmaf(pr.x, l0[u], acc0[4 * g4 + 0]);
            acc1[4 * g4 + 0] = fmaf(pr.x, l1[u], acc1[4 * g4 + 0]);
            acc0[4 * g4 + 1] = fmaf(pr.y, l0[u], acc0[4 * g4 + 1]);
            acc1[4 * g4 + 1] = fmaf(pr.y, l1[u], acc1[4 * g4 + 1]);
            acc0[4 * g4 + 2] = fmaf(pr.z, l0[u], acc0[4 * g4 + 2]);
            acc1[4 * g4 + 2] = fmaf(pr.z, l1[u], acc1[4 * g4 + 2]);
            acc0[4 * g4 + 3] = fmaf(pr.w, l0[u], acc0[4 * g4 + 3]);
            acc1[4 * g4 + 3] = fmaf(pr.w, l1[u], acc1[4 * g4 + 3]);
          }
        }
      }
    }
    __syncthreads();   // the next chunk overwrites sc and vcs
  }
  // combine the waves' partial sums, rotate back, normalise
  if (on) {
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {
      if (g < G) {
        accs[wave][g * D + 2 * lane] = acc0[g];
        accs[wave][g * D + 2 * lane + 1] = acc1[g];
      }
    }
  }
  __syncthreads();
  for (int g = wave; g < G; g += 4) {
    float y0 = 0.f, y1 = 0.f;
    if (on) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        y0 += accs[w][g * D + 2 * lane];
        y1 += accs[w][g * D + 2 * lane + 1];
      }
    }
    fwht_f32(y0, y1, lane, HALF);
    const float inv = 1.f / (static_cast<float>(D) * l_s[g]);
    if (on) {
      float2 o = make_float2(p.signs[2 * lane] * y0 * inv, p.signs[2 * lane + 1] * y1 * inv);
      *reinterpret_cast<float2*>(p.out + (row0 + g) * D + 2 * lane) = o;
    }
    if (lane == 0 && p.lse) p.lse[row0 + g] = (m_s[g] + log2f(l_s[g])) * kLn2;
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
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(n_items) * p.Hkv));
  if (head_dim == 64)
    hipExtLaunchKernelGGL(q4_decode_kernel<64>, grid, dim3(kChunk), 0, s, ev_start, ev_stop, 0, p);
  else if (head_dim == 128)
    hipExtLaunchKernelGGL(q4_decode_kernel<128>, grid, dim3(kChunk), 0, s, ev_start, ev_stop, 0, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
