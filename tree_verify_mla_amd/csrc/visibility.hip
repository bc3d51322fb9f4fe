// ddtree_compile_visibility: ancestor-or-self bitsets, positions, dense mask.
//
// One thread per tree node walks its parent chain (parents have smaller
// indices, so the walk ends at the root) and sets bit j of its row for every
// node j on the way ("The DDTree CUDA Graph Fix ...", section "The DDTree
// Architecture: Confirming Multiple-Path Evaluation").  Positions are
// prefix_len + depth ("The Architecture of a Speculative Decoding Engine
// ...", section "The Final Resolution: A Concrete Trace").  The optional
// dense byte mask is the [q_len, prefix_len + q_len] row-major layout with
// stride prefix_len + q_len ("The 30-Column Mask ...", section "Mask Stride
// Formula"); it is written from the bitsets by a second kernel.
#include "common.h"

namespace {

__global__ __launch_bounds__(64) void visibility_kernel(
    const int32_t* __restrict__ par, const int32_t* __restrict__ dep,
    const int32_t* __restrict__ qo, const int32_t* __restrict__ prefix, int W,
    uint32_t* __restrict__ bits, int64_t* __restrict__ positions) {
  const int r = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int base = qo[r];
  const int Q = qo[r + 1] - base;
  if (i >= Q) return;
  for (int w = 0; w < W; ++w) {
    uint32_t word = 0;
    int j = i;
    while (j >= 0) {
      if ((j >> 5) == w) word |= 1u << (j & 31);
      const int p = par[base + j];
      if (p >= j) break;  // malformed parent: stop the walk
      j = p;
    }
    bits[(size_t)(base + i) * W + w] = word;
  }
  if (positions) positions[base + i] = (int64_t)max(prefix[r], 0) + dep[base + i];
}

__global__ __launch_bounds__(256) void dense_mask_kernel(
    const int32_t* __restrict__ qo, const int32_t* __restrict__ prefix,
    const uint32_t* __restrict__ bits, int W, const int64_t* __restrict__ mask_indptr,
    uint8_t* __restrict__ mask) {
  const int r = blockIdx.y;
  const int i = blockIdx.x;
  const int base = qo[r];
  const int Q = qo[r + 1] - base;
  if (i >= Q) return;
  const int P = max(prefix[r], 0);
  const int len = P + Q;
  uint8_t* row = mask + mask_indptr[r] + (int64_t)i * len;
  const uint32_t* brow = bits + (size_t)(base + i) * W;
  for (int c = threadIdx.x; c < len; c += blockDim.x) {
    uint8_t v = 1;
    if (c >= P) {
      const int j = c - P;
      v = (j >> 5) < W ? (uint8_t)((brow[j >> 5] >> (j & 31)) & 1u) : (uint8_t)0;
    }
    row[c] = v;
  }
}

}  // namespace

// The bitset and position launch (arguments already checked); also used by
// ddtree_build_tree_visibility when its tree is too large for the fused builder.
int ddtree_visibility_launch(const int32_t* node_parents, const int32_t* node_depths,
                             const int32_t* qo_indptr, const int32_t* prefix_lens, int bs,
                             int max_q_len, int words_per_row, uint32_t* vis_bits,
                             int64_t* positions, hipStream_t s) {
  dim3 grid((max_q_len + 63) / 64, bs);
  hipLaunchKernelGGL(visibility_kernel, grid, dim3(64), 0, s, node_parents, node_depths,
                     qo_indptr, prefix_lens, words_per_row, vis_bits, positions);
  return ddtree::check_launch("compile_visibility");
}

extern "C" int ddtree_compile_visibility(const int32_t* node_parents, const int32_t* node_depths,
                                         const int32_t* qo_indptr, const int32_t* prefix_lens,
                                         int bs, int max_q_len, int words_per_row,
                                         uint32_t* vis_bits, int64_t* positions,
                                         uint8_t* dense_mask, const int64_t* mask_indptr,
                                         void* stream) {
  ddtree::clear_error();
  DDTREE_REQUIRE(bs >= 0, DDTREE_EINVAL, "compile_visibility: bs must be >= 0");
  if (bs == 0) return DDTREE_OK;
  DDTREE_REQUIRE(max_q_len >= 1, DDTREE_EINVAL, "compile_visibility: max_q_len must be >= 1");
  DDTREE_REQUIRE(node_parents && qo_indptr && vis_bits, DDTREE_EINVAL,
                 "compile_visibility: null required pointer");
  DDTREE_REQUIRE(!positions || (node_depths && prefix_lens), DDTREE_EINVAL,
                 "compile_visibility: positions need node_depths and prefix_lens");
  DDTREE_REQUIRE((dense_mask == nullptr) == (mask_indptr == nullptr), DDTREE_EINVAL,
                 "compile_visibility: dense_mask and mask_indptr go together");
  DDTREE_REQUIRE(!dense_mask || prefix_lens, DDTREE_EINVAL,
                 "compile_visibility: the dense mask needs prefix_lens");
  DDTREE_REQUIRE((long long)words_per_row * 32 >= max_q_len, DDTREE_EINVAL,
                 "compile_visibility: words_per_row %d < ceil(max_q_len/32) for max_q_len %d",
                 words_per_row, max_q_len);
  hipStream_t s = ddtree::as_stream(stream);
  int rc = ddtree_visibility_launch(node_parents, node_depths, qo_indptr, prefix_lens, bs,
                                    max_q_len, words_per_row, vis_bits, positions, s);
  if (rc != DDTREE_OK || !dense_mask) return rc;
  hipLaunchKernelGGL(dense_mask_kernel, dim3(max_q_len, bs), dim3(256), 0, s, qo_indptr,
                     prefix_lens, vis_bits, words_per_row, mask_indptr, dense_mask);
  return ddtree::check_launch("compile_visibility(dense)");
}
