// kv_append device work: copy-on-write block copies and the scatter of the
// new tokens' K/V into their pool slots, in one launch.
//
// The two parts touch disjoint memory, so they need no ordering between
// them: a copy reads the filled slots [0, n) of a block that several
// sequences hold (nobody writes a shared block) and writes slots [0, n) of a
// fresh block, while every new token lands at slot n or later of its block
// (append-only cache: Trellis page, section "LLM prefill and KV cache";
// copy-on-write: Dendrite page, glossary).
//
// Work unit: one 16-byte (8 x bf16) chunk, so every global access is a
// 128-bit load or store and consecutive lanes touch consecutive chunks of a
// head_dim row.  Grid-stride loop over [writes | copies].
#include "../kernels.hpp"
#include "common.hpp"

namespace pkv {
namespace {

__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  const int32_t cpr = p.D / 8;  // 16-byte chunks per head_dim row
  const int64_t n_write = static_cast<int64_t>(p.L) * p.n_rows * p.Hkv * cpr;
  const int64_t n_copy = static_cast<int64_t>(p.n_cow) * p.L * 2 * p.Hkv * p.B * cpr;
  const int64_t total = n_write + n_copy;
  const int64_t head_tile = static_cast<int64_t>(p.B) * p.D;      // one (block, head)
  const int64_t block_elems = head_tile * p.Hkv;                   // one block of one layer
  const int64_t layer_elems = block_elems * p.N;
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; u < total;
       u += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    if (u < n_write) {
      const int32_t c = static_cast<int32_t>(u % cpr);
      int64_t r = u / cpr;
      const int32_t hh = static_cast<int32_t>(r % p.Hkv);
      r /= p.Hkv;
      const int32_t row = static_cast<int32_t>(r % p.n_rows);
      const int32_t l = static_cast<int32_t>(r / p.n_rows);
      const int64_t src = ((static_cast<int64_t>(l) * p.n_rows + row) * p.Hkv + hh) * p.D + c * 8;
      const int32_t slot = p.slots[row];
      const int32_t blk = slot >> p.log2B;
      const int32_t off = slot & (p.B - 1);
      const int64_t dst = l * layer_elems + blk * block_elems + hh * head_tile +
                          static_cast<int64_t>(off) * p.D + c * 8;
      *reinterpret_cast<uint4*>(p.k_pool + dst) = *reinterpret_cast<const uint4*>(p.k_new + src);
      *reinterpret_cast<uint4*>(p.v_pool + dst) = *reinterpret_cast<const uint4*>(p.v_new + src);
    } else {
      int64_t r = u - n_write;
      const int32_t c = static_cast<int32_t>(r % cpr);
      r /= cpr;
      const int32_t slot = static_cast<int32_t>(r % p.B);
      r /= p.B;
      const int32_t hh = static_cast<int32_t>(r % p.Hkv);
      r /= p.Hkv;
      const int32_t kv = static_cast<int32_t>(r % 2);
      r /= 2;
      const int32_t l = static_cast<int32_t>(r % p.L);
      const int32_t ci = static_cast<int32_t>(r / p.L);
      const int32_t src_blk = p.cow[3 * ci + 0];
      const int32_t dst_blk = p.cow[3 * ci + 1];
      const int32_t filled = p.cow[3 * ci + 2];
      if (slot >= filled) continue;
      const int64_t within = hh * head_tile + static_cast<int64_t>(slot) * p.D + c * 8;
      uint16_t* pool = kv ? p.v_pool : p.k_pool;
      const int64_t base = l * layer_elems;
      *reinterpret_cast<uint4*>(pool + base + dst_blk * block_elems + within) =
          *reinterpret_cast<const uint4*>(pool + base + src_blk * block_elems + within);
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendParams& p, hipStream_t s) {
  const int64_t cpr = p.D / 8;
  const int64_t total = static_cast<int64_t>(p.L) * p.n_rows * p.Hkv * cpr +
                        static_cast<int64_t>(p.n_cow) * p.L * 2 * p.Hkv * p.B * cpr;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(append_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace pkv
