// bf16 verify attention on gfx950 matrix cores.
//
// Workgroup = NW wavefronts = one tile of 16*NW query rows of one request.
// Waves pair up: both waves of pair g own the same 32 query rows; wave half
// h contracts latent features [288h, 288h+288) of the score and produces
// output features [256h, 256h+256).  The tile walks its KV columns in
// blocks of 32; each block is gathered once from the slot pool into LDS and
// shared by all rows -- the prefix is read once for every tree node and head
// ("The DDTree CUDA Graph Fix ...", section "The DDTree Architecture:
// Confirming Multiple-Path Evaluation").
//
// Per block and wave pair (32 rows x 32 columns):
//   partial S^T[32 col x 32 row] = K[32 x 288] . Q^T[288 x 32]   18 x mfma_f32_32x32x16_bf16
//     A = latent rows from LDS (ds_read_b128), B = the wave's half of the
//     queries, kept in registers for the whole tile.  With columns as the
//     MFMA row index each lane's accumulator holds ONE query row, so the
//     row max is one cross-half exchange and the output rescale is one
//     multiplier per lane.  The two halves are summed through LDS.
//   mask: prefix columns always visible; column P + j visible iff bit j of
//     the row's ancestor bitset is set (tail blocks only).
//   online softmax in base 2 (identical in both waves); P^T rounded to bf16.
//   O^T[256 x 32 row] += V^T[256 x 32 col] . P^T                16 x mfma_f32_32x32x16_bf16
//     A = c_kv columns read transposed from LDS with ds_read_b64_tr_b16,
//     B = P^T straight from the score accumulator: the columns' order inside
//     the k dimension is permuted to match the accumulator layout, so P
//     never moves between lanes.
// Splitting the pair this way keeps each LDS byte feeding 32 rows while a
// wave needs only 72 VGPRs of queries and 128 accumulators of output.
//
// LDS: two 36 KB buffers (32 latent rows of 1152 B) plus a ring of three
// 32-entry slot-index lists.  Block b+1 streams in with
// global_load_lds_dwordx4 (global -> LDS, no registers) while block b is
// computed; its slot indices were fetched the same way one block earlier, so
// the gather never waits on an index load.
//
// gfx950 LDS has 64 four-byte banks; a b128 read is serviced 16 lanes at a
// time, a b64 (and the transposing b64) read 32 lanes at a time.  Row r's
// 16-byte chunks are XOR-swizzled inside each 128-byte group,
//   chunk' = chunk ^ h(r),  h(r) = ((r >> 1) & 1) << 2 | ((r >> 2) & 3),
// which makes both access patterns conflict-free: the K reads (16 rows, one
// chunk each) and the transposed V reads (4 rows x 4 adjacent chunks).
#include "attn_common.h"
#include "common.h"

namespace ddtree {
namespace attn {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef short __attribute__((ext_vector_type(4))) i16x4_t;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int ROWB = LATENT * 2;   // 1152 bytes per latent row
constexpr int BUFB = KB * ROWB;    // 36864 bytes per block buffer
constexpr int LOADS = BUFB / 1024; // 36 global_load_lds_dwordx4 (64 lanes x 16 B) per block
constexpr int RING_SLOT = 64 * 4;  // bytes per slot-index list (64 lanes x int32)
constexpr int XCH = 64 * 64;       // bytes per wave of score-exchange space (64 lanes x 16 f32)
constexpr int KS_HALF = 18;        // k-steps of 16 features per half of the 576-wide score
constexpr int FB_HALF = 8;         // 32-feature output blocks per half of the 512 outputs
constexpr float LN2 = 0.693147180559945309f;

__device__ inline int swz(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }

__device__ inline bf16x8_t lds_read_b128(const lds_char* base, int off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>(base + off);
}

__device__ inline bf16x4_t lds_read_tr(const lds_char* base, int off) {
  i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) i16x4_t*>(
          const_cast<lds_char*>(base + off)));
  return __builtin_bit_cast(bf16x4_t, v);
}

__device__ inline float max16(const f32x16_t& v) {
  float m = v[0];
#pragma unroll
  for (int k = 1; k < 16; ++k) m = fmaxf(m, v[k]);
  return m;
}

__device__ inline float other_half(float x) {
  // value of lane l ^ 32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(Params p) {
  constexpr int MT = 16 * NW;
  static_assert(MT == MT_BF16, "tile rows must match the schedule");
  __shared__ __attribute__((aligned(1024))) char smem[2 * BUFB + NW * XCH + 3 * RING_SLOT];
  lds_char* lds = (lds_char*)smem;  // generic -> LDS address space
  lds_char* xch = lds + 2 * BUFB;
  lds_char* ring = xch + NW * XCH;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hl = lane >> 5;
  const int pair = wave >> 1, half = wave & 1;
  const __bf16* __restrict__ qg = static_cast<const __bf16*>(p.q);
  const __bf16* __restrict__ pool = static_cast<const __bf16*>(p.pool);

  // ---- per-lane LDS offsets (layouts in the header comment) ----
  // K fragment of k-step ks: row l32, logical chunk 2*ks + hl.
  const int kbase = l32 * ROWB;
  int kin[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) kin[e] = 16 * ((2 * e + hl) ^ swz(l32));
  // V^T fragment via ds_read_b64_tr_b16: in each 16-lane group, lane c
  // supplies row (c / 4) and 4 features at 4 * (c % 4) of a 4 x 16 block.
  const int c16 = lane & 15, G = lane >> 4;
  const int vbase = (4 * hl + (c16 >> 2)) * ROWB + 8 * (c16 & 1);
  const int e0 = 2 * (G & 1) + ((c16 & 3) >> 1);
  const int hv0 = (((c16 >> 3) & 1) << 2) | (hl & 3);
  const int hv1 = (((c16 >> 3) & 1) << 2) | ((2 + hl) & 3);
  const int vin00 = 16 * (e0 ^ hv0), vin01 = 16 * ((4 + e0) ^ hv0);
  const int vin10 = 16 * (e0 ^ hv1), vin11 = 16 * ((4 + e0) ^ hv1);
  // score exchange: chunk k (4 floats) of lane l at (k * 64 + l) * 16
  lds_char* xmine = xch + wave * XCH + lane * 16;
  const lds_char* xpart = xch + (wave ^ 1) * XCH + lane * 16;

  // ---- schedule ----
  long long U = 0, Ge = 1, u0 = 0, u1 = 0;
  const int w = blockIdx.x;
  if (p.S == 0) {
    U = units_before(p.bs, p.qo, p.kvp, p.H, MT);
    if (U <= 0) return;
    Ge = effective_groups(U, gridDim.x);
    if (w >= Ge) return;
    u0 = range_begin(w, U, Ge);
    u1 = range_begin(w + 1, U, Ge);
  }

  long long u = u0;
  bool first = true;
  while (true) {
    int r, t, b_begin, b_end;
    long long slot = -1;
    Geom g;
    if (p.S == 0) {
      if (u >= u1) break;
      long long start;
      locate(u, p.qo, p.kvp, p.bs, p.H, MT, r, start);
      if (r >= p.bs) break;
      g = geom(p.qo, p.kvp, r, p.H, MT);
      const long long local = u - start;
      t = (int)(local / g.NB);
      b_begin = (int)(local % g.NB);
      const long long seg_end = min((long long)(t + 1) * g.NB, u1 - start);
      b_end = (int)(seg_end - (long long)t * g.NB);
      if (!(b_begin == 0 && b_end == g.NB)) slot = 2LL * w + (first ? 0 : 1);
      u = start + seg_end;
      first = false;
    } else {
      if (!first) break;
      first = false;
      const int S = p.S;
      const int s = w % S;
      t = (w / S) % p.T_max;
      r = w / (S * p.T_max);
      if (r >= p.bs) break;
      g = geom(p.qo, p.kvp, r, p.H, MT);
      if (t >= g.T) break;
      b_begin = (int)((long long)s * g.NB / S);
      b_end = (int)((long long)(s + 1) * g.NB / S);
      if (S > 1) slot = ((long long)r * p.T_max + t) * S + s;
    }

    // ---- this pair's 32 query rows; this wave's half of their features ----
    const int rho = t * MT + pair * 32 + l32;
    const bool row_ok = rho < g.R;
    const bool pair_live = t * MT + pair * 32 < g.R;  // same for both waves of the pair
    const int node = row_ok ? rho / p.H : g.Q - 1;
    bf16x8_t qf[KS_HALF];
    {
      const __bf16* qrow =
          qg + ((size_t)g.q0 * p.H + (row_ok ? rho : 0)) * LATENT + 8 * hl + 16 * KS_HALF * half;
#pragma unroll
      for (int k = 0; k < KS_HALF; ++k) {
        bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * k);
        if (!row_ok) v = bf16x8_t{};
        qf[k] = v;
      }
    }
    const uint32_t* vrow = p.vis + (size_t)(g.q0 + node) * p.W;

    f32x16_t o[FB_HALF];
#pragma unroll
    for (int fb = 0; fb < FB_HALF; ++fb) o[fb] = f32x16_t{};
    float m_run = -INFINITY, l_run = 0.f;

    // wave 0 fetches the slot indices of block b into ring slot b % 3
    auto issue_idx = [&](int b) {
      const int col = min(b * KB + lane, g.N - 1);
      __builtin_amdgcn_global_load_lds(
          p.kvi + g.kv0 + col,
          reinterpret_cast<__attribute__((address_space(3))) void*>(ring + (b % 3) * RING_SLOT),
          4, 0, 0);
    };
    // the waves share the 36 gathers (64 chunks of 16 B each) of block b
    auto issue_data = [&](int b, int buf) {
      const __attribute__((address_space(3))) int* idx =
          reinterpret_cast<const __attribute__((address_space(3))) int*>(ring + (b % 3) * RING_SLOT);
#pragma unroll
      for (int j = wave; j < LOADS; j += NW) {
        const int pc = j * 64 + lane;  // physical 16-byte chunk of the buffer
        const int row = pc / 72, c = pc % 72;
        const int chunk = (c & ~7) | ((c & 7) ^ swz(row));
        long long sid = idx[row];
        sid = sid < 0 ? 0 : (sid >= p.num_slots ? p.num_slots - 1 : sid);
        __builtin_amdgcn_global_load_lds(
            pool + sid * LATENT + chunk * 8,
            reinterpret_cast<__attribute__((address_space(3))) void*>(lds + buf * BUFB + j * 1024),
            16, 0, 0);
      }
    };

    __syncthreads();  // the previous segment is done with the buffers and the ring
    if (b_begin < b_end) {
      if (wave == 0) {
        issue_idx(b_begin);
        if (b_begin + 1 < b_end) issue_idx(b_begin + 1);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      issue_data(b_begin, 0);
    }

    for (int b = b_begin; b < b_end; ++b) {
      const int cur = (b - b_begin) & 1;
      __builtin_amdgcn_s_waitcnt(0);  // this wave's global->LDS copies have landed
      __syncthreads();                // ... and everyone else's
      if (wave == 0 && b + 2 < b_end) issue_idx(b + 2);
      if (b + 1 < b_end) issue_data(b + 1, cur ^ 1);
      const lds_char* buf = lds + cur * BUFB;

      // ---- partial S^T = K[:, half] Q^T[half, :], fragments two k-steps ahead ----
      f32x16_t s = f32x16_t{};
      if (pair_live) {
        const lds_char* kb0 = buf + kbase + kin[0];
        const lds_char* kb1 = buf + kbase + kin[1];
        const lds_char* kb2 = buf + kbase + kin[2];
        const lds_char* kb3 = buf + kbase + kin[3];
        const int kh = KS_HALF * half;  // first global k-step of this half
        auto kread = [&](int k) {      // k = local k-step 0..17
          const int ks = kh + k;
          const int e = ks & 3;
          const lds_char* b4 = e == 0 ? kb0 : (e == 1 ? kb1 : (e == 2 ? kb2 : kb3));
          return lds_read_b128(b4, 128 * (ks >> 2));
        };
        bf16x8_t a0 = kread(0);
        bf16x8_t a1 = kread(1);
#pragma unroll
        for (int k = 0; k < KS_HALF; k += 2) {
          bf16x8_t n0 = a0, n1 = a1;
          if (k + 2 < KS_HALF) n0 = kread(k + 2);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[k], s, 0, 0, 0);
          if (k + 3 < KS_HALF) n1 = kread(k + 3);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[k + 1], s, 0, 0, 0);
          a0 = n0;
          a1 = n1;
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          f32x4 v = {s[4 * k], s[4 * k + 1], s[4 * k + 2], s[4 * k + 3]};
          *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(xmine + k * 1024) = v;
        }
      }
      __syncthreads();  // both halves of every pair are in the exchange buffer
      if (!pair_live) continue;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(xpart + k * 1024);
        s[4 * k] += v[0];
        s[4 * k + 1] += v[1];
        s[4 * k + 2] += v[2];
        s[4 * k + 3] += v[3];
      }

      // ---- scale + mask ----
      const int cb = b * KB;
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] *= p.scale_log2;
      if (cb + KB > g.P) {
        const int jbase = cb - g.P;  // tree index of the block's column 0
        const int w0 = jbase > 0 ? (jbase >> 5) : 0;
        const uint32_t bw0 = w0 < p.W ? vrow[w0] : 0u;
        const uint32_t bw1 = w0 + 1 < p.W ? vrow[w0 + 1] : 0u;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int col = cb + 8 * (v >> 2) + 4 * hl + (v & 3);
          bool vis = col < g.N;
          const int j = col - g.P;
          if (vis && j >= 0) {
            const uint32_t word = (j >> 5) == w0 ? bw0 : bw1;
            vis = (word >> (j & 31)) & 1u;
          }
          if (!vis) s[v] = -INFINITY;
        }
      }

      // ---- online softmax (base 2) ----
      float mb = max16(s);
      mb = fmaxf(mb, other_half(mb));
      const float m_new = fmaxf(m_run, mb);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      float psum = 0.f;
      bf16x8_t pk[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = exp2f(s[v] - m_use);
        psum += e;
        pk[v >> 3][v & 7] = (__bf16)e;
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (__ballot(alpha != 1.f) != 0) {  // wave-uniform: skip when no row's max moved
#pragma unroll
        for (int fb = 0; fb < FB_HALF; ++fb) o[fb] *= alpha;
      }

      // ---- O^T[half] += V^T[half] P^T, fragments one feature block ahead ----
      {
        const int fh = 4 * half;  // (fb >> 1) offset of this half's features
        const lds_char* vb00 = buf + vbase + vin00 + 128 * fh;
        const lds_char* vb01 = buf + vbase + vin01 + 128 * fh;
        const lds_char* vb10 = buf + vbase + 8 * ROWB + vin10 + 128 * fh;
        const lds_char* vb11 = buf + vbase + 8 * ROWB + vin11 + 128 * fh;
        auto vread = [&](int fb, int k2) {  // fb = local block 0..7
          const int off = 128 * (fb >> 1) + 16 * k2 * ROWB;
          const bf16x4_t lo = lds_read_tr((fb & 1) ? vb01 : vb00, off);
          const bf16x4_t hi = lds_read_tr((fb & 1) ? vb11 : vb10, off);
          return (bf16x8_t)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        bf16x8_t c0 = vread(0, 0), c1 = vread(0, 1);
#pragma unroll
        for (int fb = 0; fb < FB_HALF; ++fb) {
          bf16x8_t n0 = c0, n1 = c1;
          if (fb + 1 < FB_HALF) n0 = vread(fb + 1, 0);
          o[fb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c0, pk[0], o[fb], 0, 0, 0);
          if (fb + 1 < FB_HALF) n1 = vread(fb + 1, 1);
          o[fb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c1, pk[1], o[fb], 0, 0, 0);
          c0 = n0;
          c1 = n1;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    // ---- write this segment (rows of the pair, features of the half) ----
    const float l_tot = l_run + other_half(l_run);
    if (row_ok && (slot >= 0 || b_begin < b_end)) {  // empty split segments still report m=-inf, l=0
      const size_t orow = (size_t)g.q0 * p.H + rho;
      const int fo = 256 * half + 4 * hl;
      if (slot < 0) {
        const float inv = 1.f / l_tot;
        __bf16* out = static_cast<__bf16*>(p.out) + orow * DV + fo;
#pragma unroll
        for (int fb = 0; fb < FB_HALF; ++fb) {
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            bf16x4_t v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(o[fb][4 * gq + e] * inv);
            *reinterpret_cast<bf16x4_t*>(out + 32 * fb + 8 * gq) = v4;
          }
        }
        if (half == 0 && hl == 0 && p.lse) p.lse[orow] = (m_run + log2f(l_tot)) * LN2;
      } else {
        float* base = p.ws + slot * slot_floats(MT);
        const int trow = pair * 32 + l32;
        float* ob = base + (size_t)trow * DV + fo;
#pragma unroll
        for (int fb = 0; fb < FB_HALF; ++fb) {
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            float4 v4 = make_float4(o[fb][4 * gq], o[fb][4 * gq + 1], o[fb][4 * gq + 2],
                                    o[fb][4 * gq + 3]);
            *reinterpret_cast<float4*>(ob + 32 * fb + 8 * gq) = v4;
          }
        }
        if (half == 0 && hl == 0) {
          base[(size_t)MT * DV + trow] = m_run;
          base[(size_t)MT * DV + MT + trow] = l_tot;
        }
      }
    }
  }
}

}  // namespace

int launch_bf16(const Params& p, int grid, hipStream_t s) {
  constexpr int NW = MT_BF16 / 16;
  hipLaunchKernelGGL(attn_bf16_kernel<NW>, dim3(grid), dim3(NW * 64), 0, s, p);
  return check_launch("verify_attn(bf16)");
}

}  // namespace attn
}  // namespace ddtree
