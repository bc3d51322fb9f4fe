// Work decomposition shared by the verify-attention kernels and the merge.
//
// Request r has R_r = Q_r * H query rows (node-major, head-minor) and
// N_r = P_r + Q_r logical KV columns.  Rows are cut into tiles of `mt` rows,
// columns into blocks of KB.  One work unit = (row tile, KV block).
//
// Two schedules:
//  * persistent (num_splits == 0): the grid's G workgroups take contiguous
//    ranges of the global unit list (requests in order, tiles in order,
//    blocks fastest).  A workgroup's range is a sequence of segments, each
//    inside one tile; a segment that covers its whole tile writes the final
//    output, any other writes a partial (O -- divided by the running sum in
//    the matrix-core kernel --, running max, running sum) into workspace
//    slot 2*w + (first segment of w ? 0 : 1).
//    The ranges are equal in cost, not in units: every tile is preceded by
//    KAPPA virtual units that stand for the cost of starting a segment
//    (loading the rows' queries, filling the block pipeline, storing the
//    output), and the virtual unit list is split evenly.  A range that
//    crosses a tile boundary, and so runs one segment more, gets about KAPPA
//    real units fewer.  Small problems use fewer workgroups (at least
//    MIN_UNITS units each).
//  * split (num_splits == S >= 1): workgroup (r, t, s) takes blocks
//    [s*NB/S, (s+1)*NB/S) of tile t; S == 1 writes final output, S > 1
//    writes slot (r * T_max + t) * S + s.
// The merge kernel combines a tile's partials by log-sum-exp ("The 30-Column
// Mask ...", section "The Context: Building a Custom Verify Attention
// Kernel": KV-split flash decoding with a partial reduction).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ddtree {
namespace attn {

constexpr int LATENT = 576;
constexpr int DV = 512;
constexpr int KB = 32;          // KV columns per work unit
constexpr int MIN_UNITS = 8;    // smallest persistent range per workgroup
constexpr int KAPPA = 8;        // virtual units ahead of every tile (cost of a segment start)
constexpr int MT_BF16 = 128;    // rows per tile, bf16 matrix-core kernel (4 waves x 32 rows)
constexpr int MT_F32 = 4;       // rows per tile, fp32 kernel
constexpr int MT_NARROW = 32;   // rows per tile, bf16 kernel for small problems
// The small-problem kernel serves bf16 calls whose 128-row work units (tile
// x KV block, host bounds) number at most NARROW_UNITS_PER_CU per compute
// unit.  Part s of every tile runs on XCD s % 8; the split count S is the
// largest that keeps one workgroup per compute unit on every XCD, but no
// larger than half the blocks (at least two blocks per part; ranges of up
// to NARROW_STEP blocks run whole, S = 1).
constexpr int NARROW_UNITS_PER_CU = 4;
constexpr int NARROW_STEP = 4;

struct Params {
  const void* q;
  const void* pool;
  long long num_slots;
  const int32_t* kvp;
  const int32_t* kvi;
  const int32_t* qo;
  const uint32_t* vis;
  int W;
  int bs;
  int H;
  int T_max;      // tiles per request upper bound (from max_q_len)
  int S;          // 0 = persistent schedule, else forced split count
  float scale_log2;
  void* out;
  float* lse;
  float* ws;      // partial slots
  // layer l (grid y) reads and writes these arrays advanced by l times the
  // stride (bytes); one layer: all zero
  long long q_lsb, pool_lsb, out_lsb, lse_lsb, ws_lsb;
  int L;          // layers (grid y)
};

// The parameters of layer blockIdx.y.  Null lse / ws stay null.
__device__ inline Params at_layer(Params p) {
  const long long l = blockIdx.y;
  p.q = static_cast<const char*>(p.q) + l * p.q_lsb;
  p.pool = static_cast<const char*>(p.pool) + l * p.pool_lsb;
  p.out = static_cast<char*>(p.out) + l * p.out_lsb;
  if (p.lse) p.lse = reinterpret_cast<float*>(reinterpret_cast<char*>(p.lse) + l * p.lse_lsb);
  if (p.ws) p.ws = reinterpret_cast<float*>(reinterpret_cast<char*>(p.ws) + l * p.ws_lsb);
  return p;
}

// floats per partial slot of the fp32 kernel: O [mt][512], m [mt], l [mt]
__host__ __device__ constexpr long long slot_floats(int mt) { return (long long)mt * (DV + 2); }
// the same for the matrix-core kernel, in float units: O / l [mt][512] in
// fp16 (scaled per row and 128-feature quarter), then m [mt], l [mt] and the
// inverse scales [4][mt] in fp32
__host__ __device__ constexpr long long slot_floats_bf16(int mt) { return (long long)mt * (DV / 2 + 2 + 4); }

// floats per partial slot of the small-problem kernel: O / l [32][512] in
// fp16 (scaled per row and 128-feature quarter), then {m, l, inverse scale,
// 0} [4 quarters][32 rows]
__host__ __device__ constexpr long long slot_floats_narrow() { return (long long)MT_NARROW * (DV / 2 + 16); }

// Split plan of the small-problem kernel from the host bounds; false when
// the call takes the 128-row kernel.  G = compute units.
struct NarrowPlan {
  int T;  // 32-row tiles per request (upper bound)
  int S;  // ranges per tile
};
inline bool narrow_plan(int bs, int H, int max_q_len, int max_kv_len, int G, NarrowPlan& np) {
  if (G <= 0 || bs < 1 || H < 1 || max_q_len < 1) return false;
  const long long nb = ((long long)max_kv_len + KB - 1) / KB;
  const long long t128 = ((long long)max_q_len * H + MT_BF16 - 1) / MT_BF16;
  if ((long long)bs * t128 * nb > (long long)NARROW_UNITS_PER_CU * G) return false;
  const long long t32 = ((long long)max_q_len * H + MT_NARROW - 1) / MT_NARROW;
  const long long tiles = (long long)bs * t32;
  long long per_xcd = (G / 8) / tiles;  // parts per tile on one XCD, one workgroup per compute unit
  if (per_xcd < 1) per_xcd = 1;
  long long S = nb <= NARROW_STEP ? 1 : (nb + 1) / 2;
  if (S > 8 * per_xcd) S = 8 * per_xcd;
  np.T = (int)t32;
  np.S = (int)S;
  return true;
}

struct Geom {
  int q0, Q, kv0, N, P, R, T, NB;
};

// geometry of a request from its offsets qo[r], qo[r+1], kvp[r], kvp[r+1]
__device__ inline Geom geom_of(int q0, int q1, int k0, int k1, int H, int mt) {
  Geom g;
  g.q0 = q0;
  g.Q = q1 - q0;
  g.kv0 = k0;
  g.N = k1 - k0;
  g.P = g.N - g.Q;
  if (g.Q < 1 || g.P < 0) {
    g.R = g.T = g.NB = 0;
  } else {
    g.R = g.Q * H;
    g.T = (g.R + mt - 1) / mt;
    g.NB = (g.N + KB - 1) / KB;
  }
  return g;
}

__device__ inline Geom geom(const int32_t* qo, const int32_t* kvp, int r, int H, int mt) {
  return geom_of(qo[r], qo[r + 1], kvp[r], kvp[r + 1], H, mt);
}

__device__ inline long long units_of(const Geom& g) { return (long long)g.T * g.NB; }
// real units, or virtual units (each tile KAPPA longer)
template <bool VIRT>
__device__ inline long long units_w(const Geom& g) {
  return (long long)g.T * (g.NB + (VIRT ? KAPPA : 0));
}

__device__ inline long long shfl_ll(long long v, int src) {
  int lo = __shfl((int)(v & 0xffffffffLL), src);
  int hi = __shfl((int)(v >> 32), src);
  return ((long long)hi << 32) | (unsigned int)lo;
}

__device__ inline long long shfl_xor_ll(long long v, int m) {
  int lo = __shfl_xor((int)(v & 0xffffffffLL), m);
  int hi = __shfl_xor((int)(v >> 32), m);
  return ((long long)hi << 32) | (unsigned int)lo;
}

__device__ inline long long shfl_up_ll(long long v, int d) {
  int lo = __shfl_up((int)(v & 0xffffffffLL), d);
  int hi = __shfl_up((int)(v >> 32), d);
  return ((long long)hi << 32) | (unsigned int)lo;
}

// Wave-cooperative (all 64 lanes call it): real (or virtual) units of
// requests [0, rmax).
template <bool VIRT = false>
__device__ inline long long units_before(int rmax, const int32_t* qo, const int32_t* kvp, int H,
                                         int mt) {
  const int lane = threadIdx.x & 63;
  long long tot = 0;
  for (int r0 = 0; r0 < rmax; r0 += 64) {
    const int r = r0 + lane;
    long long u = r < rmax ? units_w<VIRT>(geom(qo, kvp, r, H, mt)) : 0;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      int lo = __shfl_xor((int)(u & 0xffffffffLL), off);
      int hi = __shfl_xor((int)(u >> 32), off);
      u += ((long long)hi << 32) | (unsigned int)lo;
    }
    tot += u;
  }
  return tot;
}

// Wave-cooperative: request r whose real (or virtual) unit range
// [start, start + units) holds unit u (r = bs if u is past the end).
template <bool VIRT = false>
__device__ inline void locate(long long u, const int32_t* qo, const int32_t* kvp, int bs, int H,
                              int mt, int& r_out, long long& start_out) {
  const int lane = threadIdx.x & 63;
  long long base = 0;
  for (int r0 = 0; r0 < bs; r0 += 64) {
    const int r = r0 + lane;
    const long long ur = r < bs ? units_w<VIRT>(geom(qo, kvp, r, H, mt)) : 0;
    long long incl = ur;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      long long v = shfl_up_ll(incl, d);
      if (lane >= d) incl += v;
    }
    const long long chunk = shfl_ll(incl, 63);
    if (u < base + chunk) {
      const unsigned long long m = __ballot(base + incl > u);
      const int f = __ffsll((long long)m) - 1;
      r_out = r0 + f;
      start_out = base + shfl_ll(incl, f) - shfl_ll(ur, f);
      return;
    }
    base += chunk;
  }
  r_out = bs;
  start_out = base;
}

__device__ inline int effective_groups(long long U, int G) {
  long long g = U / MIN_UNITS;
  if (g < 1) g = 1;
  return (int)(g < G ? g : G);
}

// first (virtual) unit of workgroup w under the persistent schedule, V the
// virtual total
__device__ inline long long range_begin(long long w, long long V, long long Ge) { return w * V / Ge; }

// Wave-cooperative: the real unit at virtual position x (the first real unit
// at or after it: a position inside a tile's KAPPA prefix maps to the tile's
// first unit; x >= the virtual total maps to the real total U).
__device__ inline long long real_of(long long x, long long U, const int32_t* qo, const int32_t* kvp,
                                   int bs, int H, int mt) {
  int r;
  long long vstart;
  locate<true>(x, qo, kvp, bs, H, mt, r, vstart);
  r = __builtin_amdgcn_readfirstlane(r);
  if (r >= bs) return U;
  const Geom g = geom(qo, kvp, r, H, mt);
  const long long local = x - vstart;
  const long long t = local / (g.NB + KAPPA), off = local % (g.NB + KAPPA);
  const long long ustart = units_before(r, qo, kvp, H, mt);
  return ustart + t * g.NB + (off > KAPPA ? off - KAPPA : 0);
}

// workgroup whose persistent range holds virtual position x (V the total)
__device__ inline long long group_of(long long x, long long V, long long Ge) {
  return ((x + 1) * Ge + V - 1) / V - 1;
}

}  // namespace attn
}  // namespace ddtree

// Launchers (defined in verify_attn.hip / verify_attn_bf16.hip)
namespace ddtree {
namespace attn {
int launch_f32(const Params& p, int grid, hipStream_t s);
int launch_bf16(const Params& p, int grid, hipStream_t s);
int launch_merge(const Params& p, int mt, int grid_groups, int dtype, hipStream_t s);
// the small-problem kernel and, for S > 1, its merge (p.T_max = 32-row
// tiles, p.S = ranges per tile)
int launch_narrow(const Params& p, hipStream_t s);
}  // namespace attn
}  // namespace ddtree
