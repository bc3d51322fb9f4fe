// ddtree_verify_attn: host entry, the fp32 kernel and the partial merge.
//
// Attention of every (tree node, head) row over its request's prefix columns
// plus the columns of its own ancestors, in absorbed-MLA form: the score is
// the 576-wide dot product of the absorbed query with a latent row, the
// output the softmax-weighted sum of the rows' first 512 (c_kv) entries ("The
// Architecture of a Speculative Decoding Engine ...", section "The Forward
// Pass Pseudocode"; "The 30-Column Mask ...", sections "The Message: Tensor
// Shapes as Evidence" and "The Fix: Building Combined Indices").
//
// Softmax runs in base 2 on scores pre-multiplied by scale*log2(e); partial
// results keep (unnormalised O, running max m, running sum l) and merge as
//   M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  O = sum_s O_s 2^(m_s - M) / L,
//   lse = ln 2 * (M + log2 L).
#include <cmath>

#include "attn_common.h"
#include "common.h"

namespace ddtree {
namespace attn {

namespace {

constexpr float LN2 = 0.693147180559945309f;

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// fp32 path: one wavefront per query row.  Lane k owns latent entries
// k + 64j (9 of the 576 for the score, 8 of the 512 for the output).  The
// columns are taken 64 at a time: one round trip brings every column's slot
// and visibility (a lane each), then the visible columns go in groups of
// CG, all their rows' loads in flight together, and one online-softmax
// update per group (base 2, running max m, running sum l).
constexpr int CG = 16;

__global__ __launch_bounds__(256) void attn_f32_kernel(Params p_all) {
  const Params p = at_layer(p_all);
  const int S = p.S;
  const int wg = blockIdx.x;
  const int s = wg % S;
  const int t = (wg / S) % p.T_max;
  const int r = wg / (S * p.T_max);
  if (r >= p.bs) return;
  const Geom g = geom(p.qo, p.kvp, r, p.H, MT_F32);
  if (t >= g.T) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rho = t * MT_F32 + wave;
  if (rho >= g.R) return;  // this kernel has no barriers
  const int i = rho / p.H;
  const float* qrow = static_cast<const float*>(p.q) + ((size_t)g.q0 * p.H + rho) * LATENT;
  float qv[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) qv[k] = qrow[lane + 64 * k];
  const int b0 = (int)((long long)s * g.NB / S);
  const int b1 = (int)((long long)(s + 1) * g.NB / S);
  const int c0 = b0 * KB, c1 = min(b1 * KB, g.N);
  const uint32_t* vrow = p.vis + (size_t)(g.q0 + i) * p.W;
  const float* pool = static_cast<const float*>(p.pool);
  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = 0.f;
  for (int cb = c0; cb < c1; cb += 64) {
    // column cb + lane: its slot (clamped into the pool) and whether this
    // row sees it (prefix columns always, tree column P + j iff bit j of the
    // row's ancestor bitset); no load is conditional
    const int cl = cb + lane;
    long long sl = p.kvi[g.kv0 + min(cl, g.N - 1)];
    sl = sl < 0 ? 0 : (sl >= p.num_slots ? p.num_slots - 1 : sl);
    const int j = cl - g.P;
    const uint32_t word = vrow[min(max(j, 0) >> 5, p.W - 1)];
    const bool vis = cl < c1 && (j < 0 || ((j >> 5) < p.W && ((word >> (j & 31)) & 1u)));
    unsigned long long todo = __ballot(vis);
    while (todo) {
      // the next CG visible columns (a short group repeats its first)
      int col[CG];
      int cnt = 0;
#pragma unroll
      for (int u = 0; u < CG; ++u) {
        col[u] = todo ? __ffsll((long long)todo) - 1 : col[0];
        cnt += todo ? 1 : 0;
        todo &= todo - 1;
      }
      float kv[CG][9];
#pragma unroll
      for (int u = 0; u < CG; ++u) {
        const long long su = __shfl(sl, col[u]);
        const float* row = pool + su * LATENT;
#pragma unroll
        for (int k = 0; k < 9; ++k) kv[u][k] = row[lane + 64 * k];
      }
      float sv[CG];
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < CG; ++u) {
        float d = 0.f;
#pragma unroll
        for (int k = 0; k < 9; ++k) d = fmaf(qv[k], kv[u][k], d);
        sv[u] = wave_sum(d) * p.scale_log2;
        if (u < cnt) mx = fmaxf(mx, sv[u]);
      }
      const float mn = fmaxf(m, mx);
      const float alpha = exp2f(m - mn);
      l *= alpha;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] *= alpha;
#pragma unroll
      for (int u = 0; u < CG; ++u) {
        const float pw = u < cnt ? exp2f(sv[u] - mn) : 0.f;
        l += pw;
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = fmaf(pw, kv[u][k], o[k]);
      }
      m = mn;
    }
  }
  const size_t orow = (size_t)g.q0 * p.H + rho;
  if (S == 1) {
    float* out = static_cast<float*>(p.out) + orow * DV;
    const float inv = 1.f / l;
#pragma unroll
    for (int k = 0; k < 8; ++k) out[lane + 64 * k] = o[k] * inv;
    if (lane == 0 && p.lse) p.lse[orow] = (m + log2f(l)) * LN2;
  } else {
    float* base = p.ws + (((long long)r * p.T_max + t) * S + s) * slot_floats(MT_F32);
#pragma unroll
    for (int k = 0; k < 8; ++k) base[wave * DV + lane + 64 * k] = o[k];
    if (lane == 0) {
      base[MT_F32 * DV + wave] = m;
      base[MT_F32 * DV + MT_F32 + wave] = l;
    }
  }
}

// Merge of the fp32 kernel's split tiles (row-major partial slots): one
// wavefront per output row (4 rows per workgroup).  Lane l owns features 8l .. 8l+7 of the row.  The segments are
// taken MERGE_BATCH at a time: their m, l and partial-output loads are all
// issued before any is used, then folded in segment order by an online
// log-sum-exp (the order is fixed, so the result does not depend on timing).
// Rows are read and written as whole contiguous runs (2 KB of fp32 in, 1 KB
// of bf16 or 2 KB of fp32 out per row and segment).
constexpr int MERGE_ROWS = 4;   // rows per merge workgroup (= waves)
constexpr int MERGE_BATCH = 4;  // segments whose loads are in flight together

// workspace slot of segment k of tile t of request r (persistent schedule:
// workgroup w_first + k; its first segment lies in this tile exactly when its
// virtual range starts at or after the tile's virtual start vtile)
__device__ inline long long merge_slot(const Params& p, long long k, long long first_slot,
                                       long long w_first, long long vtile, long long V,
                                       long long Ge) {
  if (p.S > 0) return first_slot + k;
  const long long w = w_first + k;
  return 2 * w + (range_begin(w, V, Ge) >= vtile ? 0 : 1);
}

// The split segments of tile t of request r: their count and what
// merge_slot needs.  False when the tile needs no merge (one workgroup
// covered it and wrote the output itself).
struct MergePlan {
  long long nseg, first_slot, w_first, vtile, V, Ge;
};
__device__ inline bool merge_plan(const Params& p, int r, int t, const Geom& g, int mt, int G,
                                  MergePlan& m) {
  m.first_slot = 0, m.w_first = 0, m.vtile = 0, m.V = 1, m.Ge = 1;
  if (p.S > 0) {
    m.nseg = p.S;
    m.first_slot = ((long long)r * p.T_max + t) * p.S;
    return true;
  }
  const long long U = units_before(p.bs, p.qo, p.kvp, p.H, mt);
  if (U <= 0) return false;
  m.Ge = effective_groups(U, G);
  m.V = units_before<true>(p.bs, p.qo, p.kvp, p.H, mt);
  // the tile's virtual start; its real units follow the KAPPA prefix
  m.vtile = units_before<true>(r, p.qo, p.kvp, p.H, mt) + (long long)t * (g.NB + KAPPA);
  m.w_first = group_of(m.vtile + KAPPA, m.V, m.Ge);
  const long long w_last = group_of(m.vtile + KAPPA + g.NB - 1, m.V, m.Ge);
  m.nseg = w_last - m.w_first + 1;
  return w_last != m.w_first;
}

__global__ __launch_bounds__(64 * MERGE_ROWS) void merge_kernel(Params p_all, int mt, int G, int dtype) {
  const Params p = at_layer(p_all);
  const int groups = (mt + MERGE_ROWS - 1) / MERGE_ROWS;
  const int tile = blockIdx.x / groups, rgrp = blockIdx.x % groups;
  const int r = tile / p.T_max, t = tile % p.T_max;
  if (r >= p.bs) return;
  const Geom g = geom(p.qo, p.kvp, r, p.H, mt);
  if (t >= g.T) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = rgrp * MERGE_ROWS + wave;  // row inside the tile
  MergePlan m;
  if (!merge_plan(p, r, t, g, mt, G, m)) return;
  const long long nseg = m.nseg;
  if (t * mt + row >= g.R) return;  // after the wave-cooperative sums above
  const long long sf = slot_floats(mt);

  float M = -INFINITY, L = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (long long k0 = 0; k0 < nseg; k0 += MERGE_BATCH) {
    float ms[MERGE_BATCH], ls[MERGE_BATCH];
    float4 x0[MERGE_BATCH], x1[MERGE_BATCH];
#pragma unroll
    for (int j = 0; j < MERGE_BATCH; ++j) {
      if (k0 + j < nseg) {
        const float* base = p.ws + merge_slot(p, k0 + j, m.first_slot, m.w_first, m.vtile, m.V, m.Ge) * sf;
        ms[j] = base[(long long)mt * DV + row];
        ls[j] = base[(long long)mt * DV + mt + row];
        const float4* o = reinterpret_cast<const float4*>(base + (long long)row * DV + 8 * lane);
        x0[j] = o[0];
        x1[j] = o[1];
      }
    }
#pragma unroll
    for (int j = 0; j < MERGE_BATCH; ++j) {
      if (k0 + j >= nseg || ms[j] == -INFINITY) continue;  // a segment that saw no column
      const float Mn = fmaxf(M, ms[j]);
      const float a = M == -INFINITY ? 0.f : exp2f(M - Mn);
      const float b = exp2f(ms[j] - Mn);
      const float y[8] = {x0[j].x, x0[j].y, x0[j].z, x0[j].w, x1[j].x, x1[j].y, x1[j].z, x1[j].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] * a + y[e] * b;
      L = L * a + ls[j] * b;
      M = Mn;
    }
  }
  const float inv = 1.f / L;
  const size_t orow = (size_t)g.q0 * p.H + (size_t)t * mt + row;
  if (dtype == DDTREE_BF16) {
    typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)(acc[e] * inv);
    *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(p.out) + orow * DV + 8 * lane) = v;
  } else {
    float4* out = reinterpret_cast<float4*>(static_cast<float*>(p.out) + orow * DV + 8 * lane);
    out[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    out[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  }
  if (lane == 0 && p.lse) p.lse[orow] = (M + log2f(L)) * LN2;
}

// merge_plan for the persistent schedule in one pass over the requests (one
// global round trip instead of one per sum): the real and virtual unit
// totals, and the virtual units before request r.  Wave-cooperative.
__device__ inline bool merge_plan_fast(const Params& p, int r, int t, const Geom& g, int mt, int G,
                                       MergePlan& m) {
  if (p.S > 0) return merge_plan(p, r, t, g, mt, G, m);
  const int lane = threadIdx.x & 63;
  long long U = 0, V = 0, vb = 0;
  for (int r0 = 0; r0 < p.bs; r0 += 64) {
    const int rr = r0 + lane;
    long long u = 0, vu = 0;
    if (rr < p.bs) {
      const Geom gg = geom(p.qo, p.kvp, rr, p.H, mt);
      u = units_w<false>(gg);
      vu = units_w<true>(gg);
    }
    long long before = rr < r ? vu : 0;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      u += shfl_xor_ll(u, off);
      vu += shfl_xor_ll(vu, off);
      before += shfl_xor_ll(before, off);
    }
    U += u;
    V += vu;
    vb += before;
  }
  if (U <= 0) return false;
  m.first_slot = 0;
  m.Ge = effective_groups(U, G);
  m.V = V;
  m.vtile = vb + (long long)t * (g.NB + KAPPA);
  m.w_first = group_of(m.vtile + KAPPA, m.V, m.Ge);
  const long long w_last = group_of(m.vtile + KAPPA + g.NB - 1, m.V, m.Ge);
  m.nseg = w_last - m.w_first + 1;
  return w_last != m.w_first;
}

// Merge of the matrix-core kernel's split tiles.  That kernel stores a
// partial as O / l in fp16 (times a power-of-two scale per row and feature
// quarter, whose inverse it stores too) in its accumulators' lane layout --
// wave w's
// store (rg, fb, gp) writes 1 KB contiguously, lane l's 16 bytes holding
// features 128 w + 32 fb + 16 gp + 4 (l >> 5) .. +3 and the same + 8 of tile
// row 32 rg + (l & 31) -- and then m and l of every row in fp32.  So the 8
// runs c = 2 fb + gp of one (tile, row group rg, feature quarter w) hold
// features 16 c .. 16 c + 15 of the quarter; they are split into 8 / CPW
// parts of CPW runs, and one single-wave workgroup per part reads its runs
// (CPW loads of 1 KB per segment), so that lane l folds the segments for
// its own row with the same ordered log-sum-exp as merge_kernel, the loads
// of LANES_BATCH segments issued before any is used: segment j enters with
// the weight l_j 2^(m_j - M) (its values times their inverse scale).  The bf16 output goes through LDS and leaves
// as 32 CPW-byte row segments.  CPW = 2 spreads a small merge over twice as
// many compute units (each one reads at a bounded rate); CPW = 4 keeps
// larger merges at fewer waves; the smallest merges (fewer than 8 tiles)
// take CPW = 1 with 8 segments' loads in flight.
template <int CPW, int LANES_BATCH>
__global__ __launch_bounds__(64) void merge_lanes_kernel(Params p_all, int G) {
  static_assert(CPW == 1 || CPW == 2 || CPW == 4, "runs per wave");
  const Params p = at_layer(p_all);
  constexpr int mt = MT_BF16, RG = 4, NH = 8 / CPW;
  constexpr int STR = 32 * CPW + 16;  // bytes per staged row (padded)
  typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
  typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
  __shared__ __align__(16) char stg[32 * STR];
  const int q = blockIdx.x % (16 * NH), tile = blockIdx.x / (16 * NH);
  const int h = q % NH, rg = (q / NH) >> 2, w = (q / NH) & 3;
  const int r = tile / p.T_max, t = tile % p.T_max;
  if (r >= p.bs) return;
  const Geom g = geom(p.qo, p.kvp, r, p.H, mt);
  if (t >= g.T) return;
  MergePlan m;
  if (!merge_plan_fast(p, r, t, g, mt, G, m)) return;
  if (t * mt + 32 * rg >= g.R) return;  // a row group without live rows (its partials are not stored)
  const int lane = threadIdx.x & 63, l32 = lane & 31, hl = lane >> 5;
  const int row = 32 * rg + l32;  // tile row of this lane
  const long long sf = slot_floats_bf16(mt);
  const long long run = ((long long)(w * RG + rg) * 8 + CPW * h) * 512 + 8 * lane;  // in halves

  float M = -INFINITY, L = 0.f;
  float acc[8 * CPW];
#pragma unroll
  for (int e = 0; e < 8 * CPW; ++e) acc[e] = 0.f;
  for (long long k0 = 0; k0 < m.nseg; k0 += LANES_BATCH) {
    float ms[LANES_BATCH], ls[LANES_BATCH], us[LANES_BATCH];
    f16x8 x[LANES_BATCH][CPW];
#pragma unroll
    for (int j = 0; j < LANES_BATCH; ++j) {
      if (k0 + j < m.nseg) {
        const float* base =
            p.ws + merge_slot(p, k0 + j, m.first_slot, m.w_first, m.vtile, m.V, m.Ge) * sf;
        const float* stats = base + (long long)mt * DV / 2;
        ms[j] = stats[row];
        ls[j] = stats[mt + row];
        us[j] = stats[(2 + w) * mt + row];
        const f16x8* src = reinterpret_cast<const f16x8*>(reinterpret_cast<const _Float16*>(base) + run);
#pragma unroll
        for (int c = 0; c < CPW; ++c) x[j][c] = src[c * 64];
      }
    }
#pragma unroll
    for (int j = 0; j < LANES_BATCH; ++j) {
      if (k0 + j >= m.nseg || ms[j] == -INFINITY) continue;  // a segment that saw no column
      const float Mn = fmaxf(M, ms[j]);
      const float a = M == -INFINITY ? 0.f : exp2f(M - Mn);
      const float wj = ls[j] * exp2f(ms[j] - Mn);
      const float wv = wj * us[j];  // the stored values carry the quarter's scale
#pragma unroll
      for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[8 * c + e] = acc[8 * c + e] * a + (float)x[j][c][e] * wv;
      L = L * a + wj;
      M = Mn;
    }
  }
  const float inv = 1.f / L;
  // run CPW h + c holds features 16 (CPW h + c) + 4 hl .. +3 and + 8 of the
  // quarter
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[8 * c + 4 * half + e] * inv);
      *reinterpret_cast<bf16x4*>(stg + l32 * STR + 2 * (16 * c + 8 * half + 4 * hl)) = v;
    }
  __syncthreads();
  const size_t row0 = (size_t)g.q0 * p.H + (size_t)t * mt + 32 * rg;  // output row of tile row 32 rg
  constexpr int LPR = 2 * CPW;   // lanes of 16 bytes per staged row
  constexpr int RPI = 64 / LPR;  // rows per instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int tr = RPI * i + lane / LPR, col = lane % LPR;
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(stg + tr * STR + 16 * col);
    if (t * mt + 32 * rg + tr < g.R)
      *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(p.out) + (row0 + tr) * DV + 128 * w +
                                 16 * CPW * h + 8 * col) = v;
  }
  if (p.lse && w == 0 && h == 0 && hl == 0 && t * mt + row < g.R)
    p.lse[row0 + l32] = (M + log2f(L)) * LN2;
}

}  // namespace

int launch_f32(const Params& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL(attn_f32_kernel, dim3(grid, p.L), dim3(256), 0, s, p);
  return check_launch("verify_attn(f32)");
}

int launch_merge(const Params& p, int mt, int grid_groups, int dtype, hipStream_t s) {
  if (mt == MT_BF16) {  // the matrix-core kernel's lane-layout partials (bf16 output)
    // fewer than four waves per compute unit at 4 runs per wave: 2 runs; at
    // 2 runs: 1
    const long long tiles = (long long)p.bs * p.T_max * p.L;
    const long long cus = device_cu_count();
    if (tiles * 128 < 4LL * cus) {
      hipLaunchKernelGGL((merge_lanes_kernel<1, 8>), dim3((unsigned)(p.bs * p.T_max * 128), p.L),
                         dim3(64), 0, s, p, grid_groups);
    } else if (tiles * 32 < 4LL * cus) {
      hipLaunchKernelGGL((merge_lanes_kernel<2, 4>), dim3((unsigned)(p.bs * p.T_max * 64), p.L),
                         dim3(64), 0, s, p, grid_groups);
    } else {
      hipLaunchKernelGGL((merge_lanes_kernel<4, 4>), dim3((unsigned)(p.bs * p.T_max * 32), p.L),
                         dim3(64), 0, s, p, grid_groups);
    }
    return check_launch("verify_attn(merge)");
  }
  const long long groups = (long long)p.bs * p.T_max * ((mt + MERGE_ROWS - 1) / MERGE_ROWS);
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)groups, p.L), dim3(64 * MERGE_ROWS), 0, s, p, mt,
                     grid_groups, dtype);
  return check_launch("verify_attn(merge)");
}

static int bf16_grid() { return device_cu_count(); }

}  // namespace attn
}  // namespace ddtree

using namespace ddtree::attn;

extern "C" size_t ddtree_verify_attn_workspace_size(int bs, int num_heads, int max_q_len,
                                                    int max_kv_len, int num_splits, int dtype) {
  if (bs <= 0 || num_heads < 1 || max_q_len < 1 || max_kv_len < max_q_len || num_splits < 0)
    return 0;
  if (dtype != DDTREE_F32 && dtype != DDTREE_BF16) return 0;
  NarrowPlan np;
  if (dtype == DDTREE_BF16 && num_splits == 0 &&
      narrow_plan(bs, num_heads, max_q_len, max_kv_len, bf16_grid(), np))
    return np.S == 1 ? 0
                     : (size_t)((long long)bs * np.T * np.S * slot_floats_narrow() * (long long)sizeof(float));
  const int mt = dtype == DDTREE_BF16 ? MT_BF16 : MT_F32;
  const long long T_max = ((long long)max_q_len * num_heads + mt - 1) / mt;
  long long slots = 0;
  if (num_splits == 0) {
    if (dtype == DDTREE_BF16) slots = 2LL * bf16_grid();
  } else if (num_splits > 1) {
    slots = (long long)bs * T_max * num_splits;
  }
  const long long sf = dtype == DDTREE_BF16 ? slot_floats_bf16(mt) : slot_floats(mt);
  return (size_t)(slots * sf * (long long)sizeof(float));
}

extern "C" int ddtree_verify_attn_plan(int bs, int num_heads, int max_q_len, int max_kv_len,
                                       int num_splits, int dtype, int* tile_rows, int* splits) {
  ddtree::clear_error();
  DDTREE_REQUIRE(tile_rows && splits, DDTREE_EINVAL, "verify_attn_plan: null output");
  DDTREE_REQUIRE(bs >= 0 && num_heads >= 1 && max_q_len >= 1 && max_kv_len >= max_q_len &&
                     num_splits >= 0,
                 DDTREE_EINVAL, "verify_attn_plan: invalid sizes");
  DDTREE_REQUIRE(dtype == DDTREE_F32 || dtype == DDTREE_BF16, DDTREE_EINVAL,
                 "verify_attn_plan: unknown dtype %d", dtype);
  if (dtype == DDTREE_F32) {
    *tile_rows = MT_F32;
    *splits = num_splits == 0 ? 1 : num_splits;
    return DDTREE_OK;
  }
  const int G = bf16_grid();
  DDTREE_REQUIRE(G > 0, DDTREE_EHIP, "verify_attn_plan: cannot query the device compute units");
  NarrowPlan np;
  if (num_splits == 0 && narrow_plan(bs, num_heads, max_q_len, max_kv_len, G, np)) {
    *tile_rows = MT_NARROW;
    *splits = np.S;
  } else {
    *tile_rows = MT_BF16;
    *splits = num_splits;
  }
  return DDTREE_OK;
}

namespace {

// One call over L layers (L = 1: the single-layer entry point).  Strides are
// in elements of the respective arrays.
int verify_attn_impl(const char* fn, int L, const void* q, long long q_ls, const void* kv_pool,
                     long long kv_ls, int64_t num_slots, const int32_t* kv_indptr,
                     const int32_t* kv_indices, const int32_t* qo_indptr, const uint32_t* vis_bits,
                     int words_per_row, int bs, int num_heads, int max_q_len, int max_kv_len,
                     float scale, int dtype, void* out, long long out_ls, float* lse,
                     long long lse_ls, int num_splits, void* workspace, size_t workspace_bytes,
                     void* stream) {
  ddtree::clear_error();
  DDTREE_REQUIRE(L >= 1 && L <= 65535, DDTREE_EINVAL, "%s: num_layers must be in [1, 65535]", fn);
  DDTREE_REQUIRE(bs >= 0, DDTREE_EINVAL, "%s: bs must be >= 0", fn);
  if (bs == 0) return DDTREE_OK;
  DDTREE_REQUIRE(q && kv_pool && kv_indptr && kv_indices && qo_indptr && vis_bits && out,
                 DDTREE_EINVAL, "%s: null required pointer", fn);
  DDTREE_REQUIRE(q_ls >= 0 && kv_ls >= 0 && out_ls >= 0 && lse_ls >= 0, DDTREE_EINVAL,
                 "%s: layer strides must be >= 0", fn);
  DDTREE_REQUIRE(L == 1 || (out_ls > 0 && (!lse || lse_ls > 0)), DDTREE_EINVAL,
                 "%s: layer outputs must not overlap (zero output stride with %d layers)", fn, L);
  DDTREE_REQUIRE(num_heads >= 1, DDTREE_EINVAL, "%s: num_heads must be >= 1", fn);
  DDTREE_REQUIRE(max_q_len >= 1, DDTREE_EINVAL, "%s: max_q_len must be >= 1", fn);
  DDTREE_REQUIRE(max_kv_len >= max_q_len, DDTREE_EINVAL,
                 "%s: max_kv_len (%d) < max_q_len (%d)", fn, max_kv_len, max_q_len);
  DDTREE_REQUIRE((long long)words_per_row * 32 >= max_q_len, DDTREE_EINVAL,
                 "%s: words_per_row %d too small for max_q_len %d", fn, words_per_row, max_q_len);
  DDTREE_REQUIRE(std::isfinite(scale), DDTREE_EINVAL, "%s: scale must be finite", fn);
  DDTREE_REQUIRE(num_slots >= 1, DDTREE_EINVAL, "%s: num_slots must be >= 1", fn);
  DDTREE_REQUIRE(num_splits >= 0, DDTREE_EINVAL, "%s: num_splits must be >= 0", fn);
  DDTREE_REQUIRE(dtype == DDTREE_F32 || dtype == DDTREE_BF16, DDTREE_EINVAL,
                 "%s: unknown dtype %d", fn, dtype);
  const size_t per_layer = ddtree_verify_attn_workspace_size(bs, num_heads, max_q_len, max_kv_len,
                                                             num_splits, dtype);
  const size_t need = per_layer * (size_t)L;
  DDTREE_REQUIRE(workspace_bytes >= need && (need == 0 || workspace), DDTREE_EWORKSPACE,
                 "%s: workspace of %zu bytes given, %zu needed", fn, workspace_bytes, need);
  const int mt = dtype == DDTREE_BF16 ? MT_BF16 : MT_F32;
  const long long T_max = ((long long)max_q_len * num_heads + mt - 1) / mt;
  DDTREE_REQUIRE(T_max * bs * (num_splits > 0 ? num_splits : 1) < (1LL << 31) &&
                     T_max * bs * ((mt + MERGE_ROWS - 1) / MERGE_ROWS) < (1LL << 31) &&
                     T_max * bs * 64 < (1LL << 31),
                 DDTREE_EUNSUPPORTED, "%s: grid too large", fn);

  const long long esz = dtype == DDTREE_BF16 ? 2 : 4;
  Params p;
  p.q = q;
  p.pool = kv_pool;
  p.num_slots = num_slots;
  p.kvp = kv_indptr;
  p.kvi = kv_indices;
  p.qo = qo_indptr;
  p.vis = vis_bits;
  p.W = words_per_row;
  p.bs = bs;
  p.H = num_heads;
  p.T_max = (int)T_max;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  p.out = out;
  p.lse = lse;
  p.ws = static_cast<float*>(workspace);
  p.q_lsb = q_ls * esz;
  p.pool_lsb = kv_ls * esz;
  p.out_lsb = out_ls * esz;
  p.lse_lsb = lse_ls * (long long)sizeof(float);
  p.ws_lsb = (long long)per_layer;
  p.L = L;
  hipStream_t s = ddtree::as_stream(stream);

  if (dtype == DDTREE_F32) {
    p.S = num_splits == 0 ? 1 : num_splits;
    int rc = launch_f32(p, (int)(bs * T_max * p.S), s);
    if (rc != DDTREE_OK || p.S == 1) return rc;
    return launch_merge(p, mt, 0, dtype, s);
  }
  NarrowPlan np;
  if (num_splits == 0 && narrow_plan(bs, num_heads, max_q_len, max_kv_len, bf16_grid(), np)) {
    // few work units: 32-row tiles over a fixed split of the KV range, all
    // layers side by side on grid y
    DDTREE_REQUIRE((long long)bs * np.T * (np.S + 7 + 32) < (1LL << 31), DDTREE_EUNSUPPORTED,
                   "%s: grid too large", fn);
    p.T_max = np.T;
    p.S = np.S;
    return launch_narrow(p, s);
  }
  p.S = num_splits;
  int G;
  if (num_splits == 0) {
    G = bf16_grid();
    DDTREE_REQUIRE(G > 0, DDTREE_EHIP, "%s: cannot query the device compute units", fn);
  } else {
    G = (int)(bs * T_max * num_splits);
  }
  // Layers run side by side in one launch (grid y) when a layer's work is
  // small; when it already gives every workgroup of the persistent grid a
  // long range (at least LAYER_ALONE_UNITS units, bounded from the host
  // sizes), one launch per layer keeps each layer's working set alone in
  // the caches, which measured faster.
  constexpr long long LAYER_ALONE_UNITS = 64;
  const long long units_bound = (long long)bs * T_max * ((max_kv_len + KB - 1) / KB);
  const bool one_by_one = L > 1 && num_splits == 0 && units_bound >= LAYER_ALONE_UNITS * G;
  for (int l = 0; l < (one_by_one ? L : 1); ++l) {
    Params pl = p;
    if (one_by_one) {
      pl.L = 1;
      pl.q = static_cast<const char*>(p.q) + l * p.q_lsb;
      pl.pool = static_cast<const char*>(p.pool) + l * p.pool_lsb;
      pl.out = static_cast<char*>(p.out) + l * p.out_lsb;
      if (p.lse) pl.lse = reinterpret_cast<float*>(reinterpret_cast<char*>(p.lse) + l * p.lse_lsb);
      if (p.ws) pl.ws = reinterpret_cast<float*>(reinterpret_cast<char*>(p.ws) + l * p.ws_lsb);
    }
    int rc = launch_bf16(pl, G, s);
    if (rc == DDTREE_OK && num_splits != 1) rc = launch_merge(pl, mt, G, dtype, s);
    if (rc != DDTREE_OK) return rc;
  }
  return DDTREE_OK;
}

}  // namespace

extern "C" int ddtree_verify_attn(const void* q, const void* kv_pool, int64_t num_slots,
                                  const int32_t* kv_indptr, const int32_t* kv_indices,
                                  const int32_t* qo_indptr, const uint32_t* vis_bits,
                                  int words_per_row, int bs, int num_heads, int max_q_len,
                                  int max_kv_len, float scale, int dtype, void* out, float* lse,
                                  int num_splits, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return verify_attn_impl("verify_attn", 1, q, 0, kv_pool, 0, num_slots, kv_indptr, kv_indices,
                          qo_indptr, vis_bits, words_per_row, bs, num_heads, max_q_len, max_kv_len,
                          scale, dtype, out, 0, lse, 0, num_splits, workspace, workspace_bytes,
                          stream);
}

extern "C" size_t ddtree_verify_attn_layers_workspace_size(int num_layers, int bs, int num_heads,
                                                           int max_q_len, int max_kv_len,
                                                           int num_splits, int dtype) {
  if (num_layers < 1) return 0;
  return ddtree_verify_attn_workspace_size(bs, num_heads, max_q_len, max_kv_len, num_splits,
                                           dtype) *
         (size_t)num_layers;
}

extern "C" int ddtree_verify_attn_layers(
    int num_layers, const void* q, int64_t q_layer_stride, const void* kv_pool,
    int64_t kv_layer_stride, int64_t num_slots, const int32_t* kv_indptr,
    const int32_t* kv_indices, const int32_t* qo_indptr, const uint32_t* vis_bits,
    int words_per_row, int bs, int num_heads, int max_q_len, int max_kv_len, float scale,
    int dtype, void* out, int64_t out_layer_stride, float* lse, int64_t lse_layer_stride,
    int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  return verify_attn_impl("verify_attn_layers", num_layers, q, q_layer_stride, kv_pool,
                          kv_layer_stride, num_slots, kv_indptr, kv_indices, qo_indptr, vis_bits,
                          words_per_row, bs, num_heads, max_q_len, max_kv_len, scale, dtype, out,
                          out_layer_stride, lse, lse_layer_stride, num_splits, workspace,
                          workspace_bytes, stream);
}
