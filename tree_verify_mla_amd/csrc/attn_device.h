// Device helpers shared by the matrix-core verify-attention kernels
// (verify_attn_bf16.hip: 128-row tiles; verify_attn_narrow.hip: 32-row tiles
// for problems too small to fill the device).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "attn_common.h"

namespace ddtree {
namespace attn {
namespace dev {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef short __attribute__((ext_vector_type(4))) i16x4_t;
typedef uint32_t __attribute__((ext_vector_type(4))) u32x4_t;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int ROWB = LATENT * 2;   // 1152 bytes per latent row
constexpr int BUFB = KB * ROWB;    // 36864 bytes per gathered block of 32 rows
constexpr int KS = LATENT / 16;    // 36 score k-steps of 16 features
constexpr float LN2 = 0.693147180559945309f;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt << 4 | lgkmcnt << 8 | vmcnt[5:4] << 14)
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | (lgkm << 8) | ((vm >> 4) << 14);
}
constexpr int VM_ANY = 63;

// Workgroup barrier after an explicit wait (an s_waitcnt immediate).  The
// empty asm statements with a memory clobber keep the compiler from moving
// any memory access across the barrier (the barrier builtin alone does not
// order memory for the optimiser); they emit nothing.
template <int WAITCNT>
__device__ inline void barrier_after() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(WAITCNT);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ inline int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <int I, int N, typename F>
__device__ inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}
__device__ inline long long uni64(long long x) {
  const int lo = __builtin_amdgcn_readfirstlane((int)(x & 0xffffffffLL));
  const int hi = __builtin_amdgcn_readfirstlane((int)(x >> 32));
  return ((long long)hi << 32) | (unsigned int)lo;
}

// Every lane computed the same request geometry from the same loads; saying
// so lets the compiler keep it in scalar registers and branch on it.
__device__ inline Geom uniform(Geom g) {
  g.q0 = uni(g.q0); g.Q = uni(g.Q); g.kv0 = uni(g.kv0); g.N = uni(g.N);
  g.P = uni(g.P); g.R = uni(g.R); g.T = uni(g.T); g.NB = uni(g.NB);
  return g;
}

template <typename T>
__device__ inline T lds_ld(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(p);
}
template <typename T>
__device__ inline void lds_st(lds_char* p, const T& v) {
  *reinterpret_cast<__attribute__((address_space(3))) T*>(p) = v;
}

// ds_read_b64_tr_b16: four consecutive 16-bit rows of one column, transposed
// into the lane's register pair
__device__ inline bf16x4_t lds_read_tr(const lds_char* p) {
  i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) i16x4_t*>(const_cast<lds_char*>(p)));
  return __builtin_bit_cast(bf16x4_t, v);
}

// max of three floats without the NaN-quieting that fmaxf adds in IEEE mode
// (the scores are finite or -inf)
__device__ inline float max3(float a, float b, float c) {
  float r;
  asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ inline float other_half(float x) {
  // value of lane l ^ 32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

// Byte offsets inside a gathered block (32 latent rows x 72 chunks of 16
// bytes, stored as 36 groups of 1 KB: group 2m + h holds chunks 4m .. 4m+3 of
// rows 16h .. 16h+15, 16-byte position 4u + v of the group holds chunk
// 4m + ((v - (u >> 2)) & 3) of row 16h + u; b128 score reads and transposing
// b64 value reads are then free of bank conflicts).
//
// Score fragment of k-step j (lane l: row l & 31, chunk 2j + (l >> 5)) at
// kofs[j & 1] + 2048 (j >> 1).
__device__ inline void score_offsets(int lane, int& kofs0, int& kofs1) {
  const int l32 = lane & 31, hl = lane >> 5;
  const int u = l32 & 15;
  const int kb = 1024 * (l32 >> 4) + 64 * u;
  kofs0 = kb + 16 * ((hl + (u >> 2)) & 3);
  kofs1 = kb + 16 * ((2 + hl + (u >> 2)) & 3);
}
// Transposed value fragments of output block f (features 32f .. 32f+31),
// column half k2, row quad t at vofs[t] + 2048 f + 1024 k2: in 16-lane group
// g, lane c supplies block row 16 k2 + 8 t + 4 (l >> 5) + (c >> 2), features
// 32 f + 16 (g & 1) + 4 (c & 3) .. +3; after the transpose lane l holds
// feature 32 f + (l & 31) of rows 16 k2 + 8 t + 4 (l >> 5) + 0..3 -- the
// column order of the score accumulator's k-step k2.  The offsets include
// 2048 * 4 * quarter (features 128 quarter ..).
__device__ inline void value_offsets(int lane, int quarter, int& vofs0, int& vofs1) {
  const int hl = lane >> 5;
  const int g16 = lane >> 4, cq = lane & 15;
  const int cp = 2 * (g16 & 1) + ((cq & 3) >> 1);  // chunk inside the group's 4
  const int vb = 8192 * quarter + 64 * (4 * hl + (cq >> 2)) + 8 * (cq & 1);
  vofs0 = vb + 16 * ((cp + hl) & 3);
  vofs1 = vb + 512 + 16 * ((cp + 2 + hl) & 3);
}
// Gather: load i of the half-block h fills group 2i + h (i < 18) from byte
// gofs + 64 i of block row 16 h + (lane >> 2).  The immediate offset applies
// to the pool address and the LDS address alike, so the LDS base (M0) is
// target - 64 i = buffer + 1024 h + 1984 i.
__device__ inline int gather_row_offset(int lane) { return 16 * (((lane & 3) - (lane >> 4)) & 3); }

// Visibility of the 32 columns of block blk to one query row (bit c =
// column blk * KB + c): prefix columns always, tree column P + j iff bit j of
// the row's ancestor bitset, nothing at or past column N or past block
// b_end.  vw holds the row's first four bitset words (trees of up to 128
// nodes); longer rows read vrow.
__device__ inline uint32_t mask_word(int blk, int b_end, const Geom& g, int W, const uint32_t* vw,
                                     const uint32_t* vrow) {
  const int cb = blk * KB;
  const int ncol = g.N - cb;  // columns of the block that exist
  if (blk >= b_end || ncol <= 0) return 0u;
  const int jbase = cb - g.P;  // tree index of the block's column 0
  uint32_t m32;
  if (jbase >= 0) {
    const int w0 = jbase >> 5, sh = jbase & 31;
    uint32_t lo, hi;
    if (W <= 4) {
      lo = w0 == 0 ? vw[0] : (w0 == 1 ? vw[1] : (w0 == 2 ? vw[2] : vw[3]));
      hi = w0 == 0 ? vw[1] : (w0 == 1 ? vw[2] : (w0 == 2 ? vw[3] : 0u));
    } else {  // trees of more than 128 nodes
      lo = w0 < W ? vrow[w0] : 0u;
      hi = w0 + 1 < W ? vrow[w0 + 1] : 0u;
    }
    m32 = sh == 0 ? lo : (lo >> sh) | (hi << (32 - sh));
  } else if (jbase <= -KB) {  // prefix columns only
    m32 = 0xffffffffu;
  } else {  // prefix columns 0 .. -jbase-1, then tree nodes 0, 1, ...
    const int np = -jbase;
    m32 = (0xffffffffu >> (32 - np)) | (vw[0] << np);
  }
  if (ncol < 32) m32 &= (1u << ncol) - 1u;
  return m32;
}

}  // namespace dev
}  // namespace attn
}  // namespace ddtree
