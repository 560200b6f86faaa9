// Dense attention tiles: the work items whose query tile is a real dense
// contraction -- every node of a draft tree (CAST page, technical summary
// "Problem": the target checks the whole tree in one pass), the windows of a
// causal prefill, and a shared prefix read by many decode queries (SGLang
// RadixAttention page, measured benchmark: many branches over one parent).
//
// One workgroup runs one item for one kv head: up to 256 query rows (row
// groups x the G query heads of the kv head) in 16-row tiles, tile t held by
// wave t % W (4 waves of one tile, 8 of one, or for 256 rows 16 of one at
// head_dim 128 and 8 of two at head_dim 64; fixed per launch by its largest
// item), over the item's keys in 32-token steps.  Per step, with v_mfma_f32_16x16x32_bf16:
//   S^T = K Q^T  (A = K rows from LDS, B = the tile's Q in registers: each
//                 lane then holds 4 keys of ONE query row per 16-key half),
//   online softmax of S (lane local, two cross-row swaps per reduction),
//   O^T += V^T P^T (A = V^T from the transposing LDS read, B = P in bf16).
// The steps are software-pipelined inside each wave: step s + 1's score
// products are issued before step s's softmax, so the matrix cores work
// while the vector unit computes exponentials, and the V^T P^T products of
// step s follow.  K and V tiles go from global memory straight into LDS
// (global_load_lds_dwordx4) into a ring of four, issued two steps ahead of
// the step whose scores are formed.  (Measured on the tree-verify call: a
// ring of eight, six steps ahead, is no faster; neither the loads nor the
// vector instructions bound the step, which is a dependency chain per wave
// -- LDS operand reads, score products, max, exponentials, P V products --
// at two waves per SIMD.)
//
// P enters P V as bf16.  Its rounding (at most 2^-9 relative per weight)
// moves the output by about 2^-9 |v - o| sqrt(sum p^2) / sum p, negligible
// once a row's softmax mass is spread over many keys; a step in which some
// row still has a weight above 1/16 of that row's running sum (the first
// steps of every row, or a peaked row) adds the residual P - bf16(P) as a
// second bf16 term, which carries those weights to about 2^-17 relative.
#include <hip/hip_ext.h>

#include "wide_item.hpp"

namespace pkv {
namespace {

using dense::WideSmem;

template <int D, int W, int NT, int RING, int UNROLL>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(W == 16 ? 4 : 2))) void wide_kernel(
    const WorkItem* __restrict__ items, const int32_t* __restrict__ blocks, const RowGroup* __restrict__ groups,
    const uint16_t* __restrict__ q, int32_t stride, AttnParams p) {
  __shared__ WideSmem<D, RING> sm;
  __shared__ int32_t blk_s[kMaxItemBlocks];
  // consecutive workgroups take the kv heads of one item
  const int L = static_cast<int>(blockIdx.x);
  dense::wide_item<D, W, NT, RING, UNROLL>(L / p.Hkv, L % p.Hkv, items, blocks, groups, q, stride, p, sm, blk_s);
}

template <int D, int W, int NT>
hipError_t launch_wide_t(const AttnParams& p, dim3 grid, int32_t stride, hipStream_t s, hipEvent_t a,
                         hipEvent_t b) {
  constexpr int kRingTiles = 4;
  // unrolled by the ring (constant slots), except for the two-tile head_dim
  // 128 variant, where that costs a register spill (the sixteen-wave one
  // spills a few registers either way and is faster unrolled by the ring)
  constexpr int kUnroll = (D == 128 && NT == 2) ? 2 : kRingTiles;
  hipExtLaunchKernelGGL((wide_kernel<D, W, NT, kRingTiles, kUnroll>), grid, dim3(64 * W), 0, s, a, b, 0, p.items,
                        p.blocks, p.groups, p.q, stride, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_wide(const AttnParams& p, int32_t n_items, int32_t head_dim, int32_t stride,
                       int32_t max_rows, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop,
                       bool no_scratch) {
  if (n_items == 0) return hipSuccess;
  if (stride < 1 || stride > kMaxItemBlocks || max_rows < 1 || max_rows > 256) return hipErrorInvalidValue;
  const int64_t n_wg = static_cast<int64_t>(n_items) * p.Hkv;
  if (n_wg > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>(n_wg));
  // by the largest item: up to 64 rows four waves of one tile, up to 128
  // eight waves of one tile, else sixteen waves of one at head_dim 128 (four
  // waves per SIMD instead of two: measured on the tree-verify call, 41.6 ->
  // 38 us per launch; eight waves of two where no scratch may be used) and
  // eight waves of two at head_dim 64 (a step there has 8 load runs, fewer
  // than sixteen waves)
  if (head_dim == 64) {
    if (max_rows <= 64) return launch_wide_t<64, 4, 1>(p, grid, stride, s, ev_start, ev_stop);
    if (max_rows <= 128) return launch_wide_t<64, 8, 1>(p, grid, stride, s, ev_start, ev_stop);
    return launch_wide_t<64, 8, 2>(p, grid, stride, s, ev_start, ev_stop);
  }
  if (head_dim == 128) {
    if (max_rows <= 64) return launch_wide_t<128, 4, 1>(p, grid, stride, s, ev_start, ev_stop);
    if (max_rows <= 128) return launch_wide_t<128, 8, 1>(p, grid, stride, s, ev_start, ev_stop);
    if (no_scratch) return launch_wide_t<128, 8, 2>(p, grid, stride, s, ev_start, ev_stop);
    return launch_wide_t<128, 16, 1>(p, grid, stride, s, ev_start, ev_stop);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
