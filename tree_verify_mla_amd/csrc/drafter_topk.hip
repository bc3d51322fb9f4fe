// ddtree_drafter_topk: per-depth top-k log-probabilities of the drafter's
// logits -- the builder's input ("The DDTree CUDA Graph Fix ...", section
// "The DDTree Architecture: Confirming Multiple-Path Evaluation": from each
// depth position's hidden state the vocabulary head gives the top-k
// candidate tokens with their log-probabilities).
//
// The log-probability of token j of a row is x_j - lse, lse = log sum_i e^x_i
// over the whole vocabulary; the top k are the k largest, equal values in
// ascending token id.  lse is one constant per row, so the order is the order
// of the logits themselves, and only the k values need the subtraction.
//
// Two kernels, in the shape of a vocabulary split across ranks:
// * chunk_kernel: workgroup (row, chunk) reads CHUNK consecutive logits of
//   its row once (32 per thread, kept in registers) and writes the chunk's
//   max m_c, its sum s_c of e^(x - m_c), and its k best (value, id) by k
//   rounds of a workgroup argmax over the entries still in play;
// * merge_kernel: one wavefront per row folds the chunks in chunk order,
//   M = max m_c, S = sum_c s_c e^(m_c - M), lse = M + log S, and takes the
//   row's k best out of the chunks' candidates (the j-th best of a row is
//   among the j best of its chunk), writing x - lse and the ids.
// Everything is fp32; exponentials and the log are the hardware's.
#include <climits>

#include "common.h"

namespace {

constexpr int CT = 256;            // threads per chunk workgroup
constexpr int EPT = 32;            // logits per thread
constexpr int CHUNK = CT * EPT;    // logits per chunk
constexpr int KMAX = 32;           // largest k
constexpr int MERGE_PER_LANE = 16; // chunk candidates per lane in the merge (C * k <= 1024)

// order-preserving map of a finite fp32 to uint32 (larger value -> larger key)
__device__ inline uint32_t fkey(float f) {
  const uint32_t u = f == 0.f ? 0u : __float_as_uint(f);  // -0 ties with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// candidate key: larger value first, then smaller id; 0 = nothing
__device__ inline unsigned long long ckey(float v, int id) {
  return ((unsigned long long)fkey(v) << 32) | (uint32_t)(~(uint32_t)id);
}
__device__ inline int ckey_id(unsigned long long k) { return (int)~(uint32_t)(k & 0xffffffffu); }

__device__ inline unsigned long long wave_max_u64(unsigned long long k) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)(k & 0xffffffffu), off);
    const uint32_t hi = __shfl_xor((uint32_t)(k >> 32), off);
    const unsigned long long o = ((unsigned long long)hi << 32) | lo;
    k = o > k ? o : k;
  }
  return k;
}
__device__ inline float wave_max_f(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ inline float wave_sum_f(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// element e (0 <= e < CHUNK) of the chunk sits in thread t, register j:
//   VEC (16-byte loads of W = 16 / sizeof(T) elements): e = W t + W CT (j / W) + j % W
//   scalar loads:                                      e = t + CT j
template <typename T, bool VEC>
__device__ inline int elem_of(int t, int j) {
  if constexpr (VEC) {
    constexpr int W = 16 / (int)sizeof(T);
    return W * t + W * CT * (j / W) + j % W;
  } else {
    return t + CT * j;
  }
}

template <typename T>
__device__ inline float to_f32(T x) {
  if constexpr (sizeof(T) == 2) return (float)x;
  else return x;
}

template <typename T, bool VEC>
__global__ __launch_bounds__(CT) void chunk_kernel(const T* __restrict__ logits, int vocab, int C,
                                                   int k, float* __restrict__ ws_ms,
                                                   float* __restrict__ ws_val,
                                                   int32_t* __restrict__ ws_id) {
  __shared__ float red_f[CT / 64];
  __shared__ unsigned long long red_k[CT / 64];
  const int row = blockIdx.x / C, c = blockIdx.x % C;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const long long c0 = (long long)c * CHUNK;          // first element of the chunk in its row
  const int n = (int)min((long long)CHUNK, vocab - c0);  // elements of the chunk
  const T* src = logits + (size_t)row * vocab + c0;

  float x[EPT];
  if constexpr (VEC) {
    constexpr int W = 16 / (int)sizeof(T);
    typedef __attribute__((__vector_size__(16))) char v16;
#pragma unroll
    for (int q = 0; q < EPT / W; ++q) {
      const int e = W * t + W * CT * q;
      if (e + W <= n) {
        const v16 raw = *reinterpret_cast<const v16*>(src + e);
        const T* vals = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int i = 0; i < W; ++i) x[W * q + i] = to_f32(vals[i]);
      } else {
#pragma unroll
        for (int i = 0; i < W; ++i) x[W * q + i] = e + i < n ? to_f32(src[e + i]) : -INFINITY;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = t + CT * j;
      x[j] = e < n ? to_f32(src[e]) : -INFINITY;
    }
  }
  uint32_t live = 0;  // bit j: register j holds an element of the chunk still in play
#pragma unroll
  for (int j = 0; j < EPT; ++j)
    if (elem_of<T, VEC>(t, j) < n) live |= 1u << j;

  // chunk max and sum of e^(x - max)
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < EPT; ++j) m = fmaxf(m, x[j]);
  m = wave_max_f(m);
  if (lane == 0) red_f[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < EPT; ++j)
    if ((live >> j) & 1u) s += __expf(x[j] - m);
  s = wave_sum_f(s);
  if (lane == 0) red_f[wave] = s;
  __syncthreads();
  s = (red_f[0] + red_f[1]) + (red_f[2] + red_f[3]);
  const size_t slot = (size_t)row * C + c;
  if (t == 0) {
    ws_ms[2 * slot] = m;
    ws_ms[2 * slot + 1] = s;
  }

  // k rounds of a workgroup argmax (larger value, then smaller id); an
  // entry out of play has key 0
  unsigned long long kk[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j)
    kk[j] = ((live >> j) & 1u) ? ckey(x[j], (int)(c0 + elem_of<T, VEC>(t, j))) : 0ull;
  // (registers are only ever indexed by unrolled constants: a runtime index
  // would put the arrays in scratch memory)
  for (int r = 0; r < k; ++r) {
    unsigned long long best = 0;
    float bx = 0.f;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const bool b = kk[j] > best;
      best = b ? kk[j] : best;
      bx = b ? x[j] : bx;
    }
    const unsigned long long wbest = wave_max_u64(best);
    __syncthreads();  // the previous round's readers are done with red_k
    if (lane == 0) red_k[wave] = wbest;
    __syncthreads();
    unsigned long long g = red_k[0];
#pragma unroll
    for (int w = 1; w < CT / 64; ++w) g = red_k[w] > g ? red_k[w] : g;
    // keys are unique (ids are), so exactly one thread owns a nonzero winner
    if (g != 0) {
      if (g == best) {
        ws_val[slot * k + r] = bx;
        ws_id[slot * k + r] = ckey_id(g);
#pragma unroll
        for (int j = 0; j < EPT; ++j) kk[j] = kk[j] == g ? 0ull : kk[j];
      }
    } else if (t == 0) {  // fewer than k logits in the chunk
      ws_val[slot * k + r] = -INFINITY;
      ws_id[slot * k + r] = INT_MAX;
    }
  }
}

__global__ __launch_bounds__(64) void merge_kernel(int C, int k, const float* __restrict__ ws_ms,
                                                   const float* __restrict__ ws_val,
                                                   const int32_t* __restrict__ ws_id,
                                                   float* __restrict__ out_val,
                                                   int32_t* __restrict__ out_id) {
  const int row = blockIdx.x, lane = threadIdx.x;
  const float* ms = ws_ms + (size_t)row * C * 2;
  // M = max m_c, then S = sum_c s_c e^(m_c - M) in chunk order (64 chunks at
  // a time, each batch summed by the same fixed shuffle tree)
  float M = -INFINITY;
  for (int c = lane; c < C; c += 64) M = fmaxf(M, ms[2 * c]);
  M = wave_max_f(M);
  float S = 0.f;
  for (int c0 = 0; c0 < C; c0 += 64) {
    const int c = c0 + lane;
    S += wave_sum_f(c < C ? ms[2 * c + 1] * __expf(ms[2 * c] - M) : 0.f);
  }
  const float lse = M + __logf(S);

  // the chunks' candidates, MERGE_PER_LANE per lane (candidate i in lane i % 64)
  const int nc = C * k;
  const float* cv = ws_val + (size_t)row * nc;
  const int32_t* ci = ws_id + (size_t)row * nc;
  unsigned long long key[MERGE_PER_LANE];
  float val[MERGE_PER_LANE];
#pragma unroll
  for (int q = 0; q < MERGE_PER_LANE; ++q) {
    const int i = lane + 64 * q;
    key[q] = 0;
    val[q] = 0.f;
    if (i < nc && ci[i] != INT_MAX) {
      val[q] = cv[i];
      key[q] = ckey(val[q], ci[i]);
    }
  }
  for (int r = 0; r < k; ++r) {
    unsigned long long best = 0;
    float bv = 0.f;
#pragma unroll
    for (int q = 0; q < MERGE_PER_LANE; ++q) {
      const bool b = key[q] > best;
      best = b ? key[q] : best;
      bv = b ? val[q] : bv;
    }
    const unsigned long long g = wave_max_u64(best);
    if (g != 0 && g == best) {
      out_val[(size_t)row * k + r] = bv - lse;
      out_id[(size_t)row * k + r] = ckey_id(g);
#pragma unroll
      for (int q = 0; q < MERGE_PER_LANE; ++q) key[q] = key[q] == g ? 0ull : key[q];
    }
  }
}

}  // namespace

extern "C" size_t ddtree_drafter_topk_workspace_size(int rows, int vocab, int topk) {
  if (rows <= 0 || vocab <= 0 || topk < 1) return 0;
  const long long C = ((long long)vocab + CHUNK - 1) / CHUNK;
  return (size_t)((long long)rows * C * (2 + 2 * topk) * 4);
}

extern "C" int ddtree_drafter_topk(const void* logits, int dtype, int rows, int vocab, int topk,
                                   float* topk_logprobs, int32_t* topk_ids, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  ddtree::clear_error();
  DDTREE_REQUIRE(rows >= 0, DDTREE_EINVAL, "drafter_topk: rows must be >= 0");
  if (rows == 0) return DDTREE_OK;
  DDTREE_REQUIRE(logits && topk_logprobs && topk_ids, DDTREE_EINVAL,
                 "drafter_topk: null required pointer");
  DDTREE_REQUIRE(dtype == DDTREE_F32 || dtype == DDTREE_BF16, DDTREE_EINVAL,
                 "drafter_topk: unknown dtype %d", dtype);
  DDTREE_REQUIRE(vocab >= 1 && topk >= 1 && topk <= vocab, DDTREE_EINVAL,
                 "drafter_topk: need 1 <= topk <= vocab (topk %d, vocab %d)", topk, vocab);
  DDTREE_REQUIRE(topk <= KMAX, DDTREE_EUNSUPPORTED, "drafter_topk: topk %d above %d", topk, KMAX);
  const long long C = ((long long)vocab + CHUNK - 1) / CHUNK;
  DDTREE_REQUIRE(C * topk <= 64LL * MERGE_PER_LANE, DDTREE_EUNSUPPORTED,
                 "drafter_topk: vocab %d with topk %d exceeds %d chunk candidates", vocab, topk,
                 64 * MERGE_PER_LANE);
  DDTREE_REQUIRE((long long)rows * C < (1LL << 31), DDTREE_EUNSUPPORTED,
                 "drafter_topk: grid too large");
  const size_t need = ddtree_drafter_topk_workspace_size(rows, vocab, topk);
  DDTREE_REQUIRE(workspace && workspace_bytes >= need, DDTREE_EWORKSPACE,
                 "drafter_topk: workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  float* ws_ms = static_cast<float*>(workspace);
  float* ws_val = ws_ms + (size_t)rows * C * 2;
  int32_t* ws_id = reinterpret_cast<int32_t*>(ws_val + (size_t)rows * C * topk);
  hipStream_t s = ddtree::as_stream(stream);
  const dim3 grid((unsigned)(rows * C));
  const bool aligned = ((uintptr_t)logits & 15) == 0;
  if (dtype == DDTREE_F32) {
    const float* x = static_cast<const float*>(logits);
    if (aligned && vocab % 4 == 0)
      hipLaunchKernelGGL((chunk_kernel<float, true>), grid, dim3(CT), 0, s, x, vocab, (int)C, topk,
                         ws_ms, ws_val, ws_id);
    else
      hipLaunchKernelGGL((chunk_kernel<float, false>), grid, dim3(CT), 0, s, x, vocab, (int)C, topk,
                         ws_ms, ws_val, ws_id);
  } else {
    const __bf16* x = static_cast<const __bf16*>(logits);
    if (aligned && vocab % 8 == 0)
      hipLaunchKernelGGL((chunk_kernel<__bf16, true>), grid, dim3(CT), 0, s, x, vocab, (int)C,
                         topk, ws_ms, ws_val, ws_id);
    else
      hipLaunchKernelGGL((chunk_kernel<__bf16, false>), grid, dim3(CT), 0, s, x, vocab, (int)C,
                         topk, ws_ms, ws_val, ws_id);
  }
  int rc = ddtree::check_launch("drafter_topk(chunks)");
  if (rc != DDTREE_OK) return rc;
  hipLaunchKernelGGL(merge_kernel, dim3(rows), dim3(64), 0, s, (int)C, topk, ws_ms, ws_val, ws_id,
                     topk_logprobs, topk_ids);
  return ddtree::check_launch("drafter_topk(merge)");
}
