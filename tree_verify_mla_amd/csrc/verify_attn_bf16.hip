// bf16 verify attention on gfx950 matrix cores.
//
// Workgroup = 4 wavefronts = one tile of 128 query rows of one request.  The
// tile walks its KV columns in blocks of 32; each block is gathered once
// from the slot pool into LDS and shared by all 128 rows -- the prefix is
// read once for every tree node and head ("The DDTree CUDA Graph Fix ...",
// section "The DDTree Architecture: Confirming Multiple-Path Evaluation").
//
// Wave w does two jobs per block:
//   scores of rows 32w .. 32w+31 (its "own" rows)
//     S^T[32 col x 32 row] = K[32 x 576] . Q^T[576 x 32]      36 x mfma_f32_32x32x16_bf16
//     A = latent rows from LDS (ds_read_b128), B = the rows' queries, kept in
//     registers (144 VGPRs) for the whole tile.  With columns as the MFMA row
//     index each lane's accumulator holds ONE query row (16 of its 32
//     columns; lane l ^ 32 holds the rest), so the row max is one cross-half
//     exchange.  Mask (tail blocks only): prefix columns always visible,
//     column P + j visible iff bit j of the row's ancestor bitset is set.
//     Online softmax in base 2 in registers; P^T rounded to bf16 already has
//     the lane layout of the value MFMA's B operand (the columns' order
//     inside the k dimension is permuted to match the accumulator, and the
//     value fragments use the same permutation).  P^T and the rows' rescale
//     factors go to LDS.
//   values of output features 128w .. 128w+127 for all 128 rows
//     O^T[128 x 128 row] += V^T[128 x 32 col] . P^T[32 col x 128 row]   32 x mfma
//     A = c_kv columns read transposed from LDS (ds_read_b64_tr_b16); each
//     fragment feeds four MFMAs (one per 32-row group); B = P^T from LDS.
//     The 128 x 128 fp32 accumulator is 256 AGPRs.
// The LDS instruction rate bounds this loop together with the matrix cores:
// per wave and block it issues 36 b128 score reads, 16 transposing value
// reads and 8 b128 P^T reads.
//
// Block buffer layout.  A block is 32 latent rows x 72 chunks of 16 bytes,
// stored as 36 groups of 1 KB: group 2m + h holds chunks 4m .. 4m+3 of rows
// 16h .. 16h+15, and 16-byte position 4u + v of the group holds chunk
// 4m + ((v - (u >> 2)) & 3) of row 16h + u.
// * gather: one buffer_load_dwordx4 ... lds fills one group (lane =
//   position).  Each 4-lane quad reads one 64-byte span of one row, and
//   wave w fetches rows 16 (w & 1) + l/4, bytes [576 (w >> 1), +576) of
//   them: one pool offset per lane and block, the 64-byte steps in the
//   instruction's immediate.
// * score fragment (k-step j, lane l: row l & 31, chunk 2j + (l >> 5)): two
//   base addresses (j even / odd) plus an immediate 2 KB * (j >> 1).
// * transposed value fragments (4 rows x 16 features per 16 lanes): two
//   base addresses plus immediates.
// gfx950 LDS has 64 four-byte banks; a b128 read is serviced 16 lanes at a
// time, a b64 (and the transposing b64) read 32 lanes at a time.  The
// rotation by (u >> 2) puts the lanes of each phase of both patterns on 16
// distinct 16-byte positions mod 256 bytes, so neither has bank conflicts.
//
// Pipeline: four block buffers, two barriers per block.  Iteration b:
//   barrier  every wave is done with block b-1 and with P^T(b-1);
//   phase A  P^T(b) and the factors of the own rows to LDS; 36 score MFMAs of
//            block b+1, the gather of block b+3 and the slot-index load of
//            block b+4 spread underneath; after step SYNC_STEP:
//   barrier  P^T(b) complete, block b+2 landed for every wave; then the first
//            P^T and value fragments of block b are read under the last
//            score MFMAs;
//   phase B  rare rescale of O; 32 value MFMAs of block b; the softmax of
//            block b+1 underneath; the first score fragments of block b+2.
#include <climits>

#include "attn_common.h"
#include "attn_device.h"
#include "common.h"

namespace ddtree {
namespace attn {

namespace {

using namespace dev;

constexpr int NWAVE = 4;           // waves per workgroup, 32 own rows each
constexpr int LOADS = BUFB / 1024; // 36 one-KB groups per block
constexpr int LPW = LOADS / NWAVE; // gather loads per wave per block
constexpr int NBUF = 4;            // block buffers (a power of two)
constexpr int RG = 4;              // 32-row groups of the tile
constexpr int FB = 4;              // 32-feature output blocks per wave
constexpr int KDEPTH = 4;          // score fragments read ahead
constexpr int SYNC_STEP = 28;      // score step before which the mid-block barrier sits
constexpr int PBUF = NBUF * BUFB;            // P^T of a block: [row group][k-step] x 1 KB
constexpr int ABUF = PBUF + RG * 2 * 1024;   // rescale factors [32][RG] f32
constexpr int SBUF = ABUF + 32 * RG * 4;     // final m, l [2][32][RG] f32
constexpr int TABB = SBUF + 2 * 32 * RG * 4;  // request table: int [4][64], long long [2][64]
constexpr int TAB_REQ = 64;                  // requests the table holds
constexpr int LDS_BYTES = TABB + 4 * TAB_REQ * 4 + 2 * TAB_REQ * 8;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
static_assert(3 * (LPW - 1) + 1 < SYNC_STEP, "gathers are issued before the mid-block barrier");

// Register files.  The 256 output accumulators fill the AGPRs; the score
// accumulator, which the softmax reads, lives in VGPRs with the queries and
// everything else.  The score MFMAs are builtins compiled in VGPR form
// (-mllvm -amdgpu-mfma-vgpr-form), so the compiler sees them and pads every
// hazard around them, copies included.  The value MFMAs are inline asm on
// AGPR operands ("a"): only the next value MFMA on the same accumulator reads
// their result (back-to-back accumulation needs no wait), and code that
// touches the accumulators otherwise -- the rare rescale and the epilogue --
// first waits out the result hazard of an 8-pass MFMA (value_drain), and the
// rescale leaves 2+ wait states before the next MFMA reads what it wrote.
// Their A and B operands come straight from LDS reads, covered by the
// compiler's wait counts (which see inline-asm operands).
__device__ inline void value_mfma(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ inline void value_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }
__device__ inline void in_agprs(f32x16_t& x) { asm volatile("" : "+a"(x)); }
// The softmax's arithmetic is pure as well: an empty asm that takes a
// stage's result keeps the stage under the MFMA it was placed beneath.
template <typename T>
__device__ inline void here(T& x) {
  asm volatile("" : "+v"(x));
}
// BUF: the pool is addressed through a buffer resource (32-bit offsets,
// pools under 4 GiB).  The gathers are then buffer_load ... lds, which the
// compiler's wait-count tracking keeps apart from LDS reads, so the LDS
// reads of fragments wait only for themselves.  With global_load_lds (the
// form for larger pools) every LDS read waits for all outstanding LDS
// traffic.
template <bool BUF>
__global__ __launch_bounds__(NWAVE * 64) void attn_bf16_kernel(Params p_all) {
  // The body uses buffer-resource builtins that exist only for the device;
  // the host pass needs nothing but the kernel's symbol.
#if defined(__HIP_DEVICE_COMPILE__)
  const Params p = at_layer(p_all);
  constexpr int MT = 32 * NWAVE;
  static_assert(MT == MT_BF16, "tile rows must match the schedule");
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
  lds_char* lds = (lds_char*)smem;  // generic -> LDS address space

  const int lane = threadIdx.x & 63;
  const int wave = uni(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const __bf16* __restrict__ qg = static_cast<const __bf16*>(p.q);
  const char* __restrict__ poolb = static_cast<const char*>(p.pool);
  const __amdgpu_buffer_rsrc_t pool_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.pool), 0, (int)(unsigned)min((long long)p.num_slots * ROWB, 0xffffffffLL),
      0x00020000);  // gfx9 raw buffer: untyped, no swizzle

  // ---- lane constants of the buffer layout (header comment) ----
  int kofs0, kofs1;  // score fragment of k-step j at kofs[j & 1] + 2048 (j >> 1)
  score_offsets(lane, kofs0, kofs1);
  // value fragments of global output block f at vofs[t] + 2048 f + 1024 k2;
  // this wave's blocks are f = 4 wave + fb
  int vofs0, vofs1;
  value_offsets(lane, wave, vofs0, vofs1);
  // gather: the block row this lane fetches and its byte offset in the row
  const int grow = 16 * (wave & 1) + (lane >> 2);
  const int gofs = gather_row_offset(lane) + 576 * (wave >> 1);
  // Load i of a block fills group 2 (9 (wave >> 1) + i) + (wave & 1) from
  // row offset gofs + 64 i.  The immediate offset applies to the pool address
  // and the LDS address alike, so the LDS base (M0) is target - 64 i.
  const int wofs = 18432 * (wave >> 1) + 1024 * (wave & 1);
  // P^T fragment (row group rg, k-step k2) at 2 KB rg + 1 KB k2, 16 bytes per
  // lane; rescale factor of tile row 32 rg + r at 16 r + 4 rg; final m and l
  // likewise (l 512 bytes further)
  lds_char* const pbuf = lds + PBUF;
  lds_char* const abuf = lds + ABUF;
  lds_char* const sbuf = lds + SBUF;
  const int pofs = 16 * lane;

  // ---- schedule ----
  // Persistent: G workgroups take equal contiguous ranges of the unit list.
  // Workgroup w runs on XCD w % 8 (hardware round-robin), so ranges are
  // handed out by "virtual" id v = (w % 8) * (G / 8) + w / 8: the workgroups
  // of one XCD share a contiguous stretch of work -- for the 64-head batch
  // one request -- and re-read its KV blocks from that XCD's L2 instead of
  // the last-level cache.
  //
  // With at most TAB_REQ requests, wave 0 first reads every request's offsets
  // once (one memory round trip) and puts them, with the running sums of the
  // requests' real and virtual units, in an LDS table; every later lookup
  // (the range's ends, each segment's request and geometry) is then a table
  // read and a ballot instead of a chain of dependent global reads.
  const bool table = p.S == 0 && p.bs <= TAB_REQ;
  lds_char* const tab_i = lds + TABB;                    // q0, q1, k0, k1 of request r
  lds_char* const tab_u = lds + TABB + 4 * TAB_REQ * 4;  // inclusive real, virtual units
  if (table) {
    if (wave == 0) {
      const bool in = lane < p.bs;
      const int q0 = in ? p.qo[lane] : 0, q1 = in ? p.qo[lane + 1] : 0;
      const int k0 = in ? p.kvp[lane] : 0, k1 = in ? p.kvp[lane + 1] : 0;
      const Geom gg = geom_of(q0, q1, k0, k1, p.H, MT);
      long long ui = in ? units_w<false>(gg) : 0, vi = in ? units_w<true>(gg) : 0;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const long long a = shfl_up_ll(ui, d), b = shfl_up_ll(vi, d);
        if (lane >= d) {
          ui += a;
          vi += b;
        }
      }
      lds_st(tab_i + 4 * lane, q0);
      lds_st(tab_i + 4 * TAB_REQ + 4 * lane, q1);
      lds_st(tab_i + 8 * TAB_REQ + 4 * lane, k0);
      lds_st(tab_i + 12 * TAB_REQ + 4 * lane, k1);
      lds_st(tab_u + 8 * lane, ui);
      lds_st(tab_u + 8 * TAB_REQ + 8 * lane, vi);
    }
    barrier_after<waitcnt_imm(VM_ANY, 0)>();
  }
  // geometry of request r (uniform) from the table or from memory
  auto req_geom = [&](int r) {
    if (!table) return uniform(geom(p.qo, p.kvp, r, p.H, MT));
    return uniform(geom_of(lds_ld<int>(tab_i + 4 * r), lds_ld<int>(tab_i + 4 * TAB_REQ + 4 * r),
                           lds_ld<int>(tab_i + 8 * TAB_REQ + 4 * r),
                           lds_ld<int>(tab_i + 12 * TAB_REQ + 4 * r), p.H, MT));
  };
  // the request whose real (VIRT: virtual) unit range holds unit x and the
  // units before it (r = bs and the total past the end), as locate()
  auto req_locate = [&](long long x, bool virt, int& r_out, long long& start_out) {
    const long long inc = lane < p.bs ? lds_ld<long long>(tab_u + (virt ? 8 * TAB_REQ : 0) + 8 * lane) : 0;
    const unsigned long long m = __ballot(lane < p.bs && inc > x);
    const long long tot = shfl_ll(inc, p.bs - 1);
    if (m == 0) {
      r_out = p.bs;
      start_out = tot;
    } else {
      const int f = __ffsll((long long)m) - 1;
      r_out = f;
      start_out = f == 0 ? 0 : shfl_ll(inc, f - 1);
    }
  };
  long long U = 0, V = 0, Ge = 1, u0 = 0, u1 = 0, v = blockIdx.x;
  if (p.S == 0) {
    if (table) {
      int rr;
      req_locate(LLONG_MAX - 1, false, rr, U);
      req_locate(LLONG_MAX - 1, true, rr, V);
      U = uni64(U);
      V = uni64(V);
    } else {
      U = uni64(units_before(p.bs, p.qo, p.kvp, p.H, MT));
      V = uni64(units_before<true>(p.bs, p.qo, p.kvp, p.H, MT));
    }
    if (U <= 0) return;
    Ge = effective_groups(U, gridDim.x);
    if (blockIdx.x >= Ge) return;
    if (Ge == gridDim.x && (Ge & 7) == 0) v = (blockIdx.x & 7) * (Ge >> 3) + (blockIdx.x >> 3);
    // equal shares of the virtual unit list (segment starts cost KAPPA units);
    // real_of: the real unit at virtual position x (a position inside a
    // tile's KAPPA prefix maps to the tile's first unit)
    auto real_at = [&](long long x) -> long long {
      if (!table) return uni64(real_of(x, U, p.qo, p.kvp, p.bs, p.H, MT));
      int r;
      long long vstart;
      req_locate(x, true, r, vstart);
      r = uni(r);
      if (r >= p.bs) return U;
      vstart = uni64(vstart);
      const Geom gr = req_geom(r);
      const long long local = x - vstart;
      const long long tt = local / (gr.NB + KAPPA), off = local % (gr.NB + KAPPA);
      // units of the requests before r: the inclusive sum of r - 1
      const long long inc = lane < p.bs ? lds_ld<long long>(tab_u + 8 * lane) : 0;
      const long long ustart = r == 0 ? 0 : shfl_ll(inc, r - 1);
      return uni64(ustart + tt * gr.NB + (off > KAPPA ? off - KAPPA : 0));
    };
    u0 = real_at(range_begin(v, V, Ge));
    u1 = real_at(range_begin(v + 1, V, Ge));
    if (u0 >= u1) return;  // a share that holds no real unit
  }

  // A range is a run of segments, each inside one tile.  Only the first can
  // start mid-tile; it runs last, so every workgroup sweeps its tiles' KV
  // blocks from block 0 onward in step with the rest of its XCD.
  long long cursor = 0;  // next unit among the segments after the first
  bool first_done = false;
  auto seg_locate = [&](long long u, int& r_out, long long& start_out) {
    if (table) {
      req_locate(u, false, r_out, start_out);
    } else {
      locate(u, p.qo, p.kvp, p.bs, p.H, MT, r_out, start_out);
    }
    r_out = uni(r_out);
    start_out = uni64(start_out);
  };
  if (p.S == 0) {
    int r0;
    long long start0;
    seg_locate(u0, r0, start0);
    if (r0 >= p.bs) return;
    const Geom g0 = req_geom(r0);
    cursor = start0 + min(((u0 - start0) / g0.NB + 1) * g0.NB, u1 - start0);
  }
  int seg_no = 0;
  const int nslot_m1 = (int)min(p.num_slots - 1, (long long)0x7fffffff);
  const float c = p.scale_log2;
  while (true) {
    int r, t, b_begin, b_end;
    long long slot = -1;
    Geom g;
    if (p.S == 0) {
      long long useg;
      if (cursor < u1) {
        useg = cursor;
      } else if (!first_done) {
        useg = u0;
        first_done = true;
      } else {
        break;
      }
      long long start;
      seg_locate(useg, r, start);
      if (r >= p.bs) break;
      g = req_geom(r);
      const long long local = useg - start;
      t = uni((int)(local / g.NB));
      b_begin = uni((int)(local % g.NB));
      const long long seg_end = min((long long)(t + 1) * g.NB, u1 - start);
      b_end = uni((int)(seg_end - (long long)t * g.NB));
      if (!(b_begin == 0 && b_end == g.NB)) slot = 2 * v + (useg == u0 ? 0 : 1);
      if (useg != u0) cursor = start + seg_end;
    } else {
      if (seg_no > 0) break;
      const int S = p.S;
      const int s = blockIdx.x % S;
      t = (blockIdx.x / S) % p.T_max;
      r = blockIdx.x / (S * p.T_max);
      if (r >= p.bs) break;
      g = uniform(geom(p.qo, p.kvp, r, p.H, MT));
      if (t >= g.T) break;
      b_begin = uni((int)((long long)s * g.NB / S));
      b_end = uni((int)((long long)(s + 1) * g.NB / S));
      if (S > 1) slot = ((long long)r * p.T_max + t) * S + s;
    }
    ++seg_no;

    // ---- this wave's own 32 query rows ----
    // Loads are issued in the order their results are needed, since a wave's
    // loads complete in order: the row's ancestor bitset words and the slots
    // of the first blocks, then the queries, which the gathers need not wait
    // for.
    const int rho = t * MT + wave * 32 + l32;
    const bool row_ok = rho < g.R;
    // A row past the tile's end (a wave may hold only such rows) still runs
    // the whole pipeline, on the queries of the request's row 0, so that every
    // wave follows one straight-line path; the epilogue writes only rows < R.
    const int node = row_ok ? rho / p.H : g.Q - 1;
    // The row's ancestor bitset words, read once per segment: a global load
    // inside the block loop would have to wait behind the in-flight gathers.
    // Rows of up to 128 tree nodes keep all words in registers; words past
    // the row's W (repeats of its last word) only ever reach columns past the
    // tree, which the mask clears by position.  No load here is conditional:
    // the compiler's wait counting through branches would wait for all of
    // them at once.
    long long qoff = ((long long)g.q0 * p.H + (row_ok ? rho : 0)) * LATENT + 8 * hl;
    asm volatile("" : "+v"(qoff));  // address formed before the loads are issued
    const __bf16* qrow = qg + qoff;
    const uint32_t* vrow = p.vis + (size_t)(g.q0 + node) * p.W;
    uint32_t vw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) vw[k] = vrow[min(k, p.W - 1)];
    // slot of the block row this lane gathers in block b (clamped to the
    // request's last column: blocks past the end gather a valid row)
    const int32_t* kvi = p.kvi + g.kv0;
    auto load_idx = [&](int b) { return kvi[min(b * KB + grow, g.N - 1)]; };
    int idx_pro[4];  // slots of blocks b_begin .. b_begin+3
#pragma unroll
    for (int k = 0; k < 4; ++k) idx_pro[k] = load_idx(b_begin + k);
    bf16x8_t qf[KS];  // B operand of k-step j: features 16 j + 8 hl .. +7 of row l32
#pragma unroll
    for (int k = 0; k < KS; ++k) qf[k] = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * k);

    f32x16_t o[RG][FB];  // O^T: row group rg, features 128 wave + 32 fb .. +31
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        o[rg][fb] = f32x16_t{};
        in_agprs(o[rg][fb]);
      }

    auto gather_src = [&](int sid) {
      // The index is opaque here so that the clamp below (and with it the
      // wait for the index load) cannot be hoisted to the load itself.
      asm volatile("" : "+v"(sid));
      sid = min(max(sid, 0), nslot_m1);
      if constexpr (BUF)
        return (int)((unsigned)sid * ROWB + gofs);  // byte offset in the pool
      else
        return poolb + (long long)sid * ROWB + gofs;
    };
    // LDS base of this wave's gather into buffer dst (wave-uniform, so M0 is
    // formed with scalar adds)
    auto gather_base = [&](const lds_char* dst) { return uni((int)(size_t)dst + wofs); };
    auto gather_one = [&](int base, auto src, auto ic) {
      constexpr int i = decltype(ic)::value;
      auto* d = (__attribute__((address_space(3))) void*)(size_t)(base + 1984 * i);
      if constexpr (BUF)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(pool_rsrc, d, 16, src, 0, 64 * i, 0);
      else
        __builtin_amdgcn_global_load_lds(src, d, 16, 64 * i, 0);
    };
    auto issue_data = [&](const lds_char* dst, int sid) {
      const auto src = gather_src(sid);
      const int base = gather_base(dst);
      static_for<0, LPW>([&](auto ic) { gather_one(base, src, ic); });
    };

    // visibility of block blk's 32 columns to this lane's row
    auto mask_word = [&](int blk) -> uint32_t { return dev::mask_word(blk, b_end, g, p.W, vw, vrow); };

    // ------------------------------------------------------------------
    // Softmax of one block of the own rows, in stages (each sits under one
    // value MFMA).  Lane l holds columns 8 (x >> 2) + 4 (l >> 5) + (x & 3),
    // x = 0..15, of row l & 31; x = 0..7 is k-step 0 of the value product,
    // 8..15 k-step 1.  The reference m moves lazily: only when the block max
    // exceeds it by RESCALE_SLACK (log2 units), so the rescale of O is rare
    // and weights stay below 2^RESCALE_SLACK.  O and l share the reference,
    // so the result is exact.  The row sum adds the fp32 weights (the value
    // product takes them rounded to bf16).
    // ------------------------------------------------------------------
    constexpr float RESCALE_SLACK = 8.f;
    float m_run = -INFINITY;  // reference of the lane's row (same in lanes l and l ^ 32)
    float l_run = 0.f;        // sum of the lane's 16 columns' weights
    float mb = 0.f, mu = 0.f, alpha = 1.f;
    auto sm_mask = [&](f32x16_t& s, int blk) {
      const uint32_t mine = mask_word(blk) >> (4 * hl);
#pragma unroll
      for (int x = 0; x < 16; ++x)
        if (!((mine >> (8 * (x >> 2) + (x & 3))) & 1u)) s[x] = -INFINITY;
      here(s);
    };
    auto sm_max0 = [&](const f32x16_t& s) {
      mb = max3(max3(s[0], s[1], s[2]), max3(s[3], s[4], s[5]), max3(s[6], s[7], s[8]));
      here(mb);
    };
    auto sm_max1 = [&](const f32x16_t& s) {
      mb = max3(max3(s[9], s[10], s[11]), max3(s[12], s[13], s[14]), max3(s[15], mb, mb));
      here(mb);
    };
    // the new reference, in three dependent stages
    float m_new = 0.f;
    auto sm_ref1 = [&]() {
      mb = fmaxf(mb, other_half(mb)) * c;  // c > 0
      here(mb);
    };
    auto sm_ref2 = [&]() {
      const bool move = mb > m_run + RESCALE_SLACK;  // also true while m_run is -inf
      m_new = move ? mb : m_run;
      // rows that keep their reference get exactly 1 (also when it is still -inf)
      alpha = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      here(m_new);
      here(alpha);
    };
    auto sm_ref3 = [&]() {
      l_run *= alpha;
      m_run = m_new;
      mu = m_run == -INFINITY ? 0.f : m_run;  // all columns masked so far
      here(mu);
      here(l_run);
    };
    // weight of column x under the reference; the weights of columns x - 1
    // and x (x odd) go out as one packed bf16 pair, pw[x >> 1]
    uint32_t pw[8];
    float e_even = 0.f;
    auto sm_exp = [&](const f32x16_t& s, auto xc) {
      constexpr int x = decltype(xc)::value;
      const float e = __builtin_amdgcn_exp2f(fmaf(s[x], c, -mu));
      l_run += e;
      here(l_run);
      if constexpr (x & 1) {
        const bf16x2_t two = {(__bf16)e_even, (__bf16)e};
        pw[x >> 1] = __builtin_bit_cast(uint32_t, two);
        here(pw[x >> 1]);
      } else {
        e_even = e;
        here(e_even);
      }
    };
    auto sm_pack = [&](bf16x8_t& pk0, bf16x8_t& pk1) {
      pk0 = __builtin_bit_cast(bf16x8_t, u32x4_t{pw[0], pw[1], pw[2], pw[3]});
      pk1 = __builtin_bit_cast(bf16x8_t, u32x4_t{pw[4], pw[5], pw[6], pw[7]});
    };

    auto score_mfmas = [&](const lds_char* kbuf, bf16x8_t* kf, auto&& under) {
      // S^T of one block; under(k) runs beneath step k
      const lds_char* kb0 = kbuf + kofs0;
      const lds_char* kb1 = kbuf + kofs1;
      f32x16_t acc;
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, KS>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        under(kc);
        if constexpr (k + KDEPTH < KS)
          kf[k + KDEPTH] = lds_ld<bf16x8_t>(((k + KDEPTH) & 1 ? kb1 : kb0) + 2048 * ((k + KDEPTH) >> 1));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[k], qf[k], k == 0 ? f32x16_t{} : acc, 0, 0, 0);
        here(acc);  // keeps the (pure) MFMA at its step
        __builtin_amdgcn_sched_barrier(0);
      });
      return acc;
    };
    auto kprefetch = [&](const lds_char* kbuf, bf16x8_t* kf) {
#pragma unroll
      for (int k = 0; k < KDEPTH; ++k)
        kf[k] = lds_ld<bf16x8_t>((k & 1 ? kbuf + kofs1 : kbuf + kofs0) + 2048 * (k >> 1));
    };

    // ------------------------------------------------------------------
    // Prologue: gather blocks b0 .. b0+2, the scores and softmax of b0
    // (P^T(b0) of the own rows), and the first score fragments of b0+1.
    // ------------------------------------------------------------------
    // the previous segment is done with all of LDS (its output stores and
    // this segment's loads above may still be in flight)
    barrier_after<waitcnt_imm(VM_ANY, 0)>();
    bf16x8_t kpre[KDEPTH];  // first score fragments of the next block
#pragma unroll
    for (int k = 0; k < KDEPTH; ++k) kpre[k] = bf16x8_t{};
    bf16x8_t pc0 = bf16x8_t{}, pc1 = bf16x8_t{};  // own rows' P^T of the current block
    int idx_cur = 0;  // slot for the gather of block b+3
    if (b_begin < b_end) {
      const int b0 = b_begin;
      // The pipeline is straight-line: blocks past the segment's end are
      // "gathered" too (a valid row, into a buffer nobody reads), so every
      // wait below is one fixed count.
      issue_data(lds + (b0 & (NBUF - 1)) * BUFB, idx_pro[0]);
      issue_data(lds + ((b0 + 1) & (NBUF - 1)) * BUFB, idx_pro[1]);
      issue_data(lds + ((b0 + 2) & (NBUF - 1)) * BUFB, idx_pro[2]);
      idx_cur = idx_pro[3];
      barrier_after<waitcnt_imm(LPW, 0)>();  // blocks b0, b0+1 (and the queries) have landed
      bf16x8_t kf[KS];
      kprefetch(lds + (b0 & (NBUF - 1)) * BUFB, kf);
      f32x16_t s0 = score_mfmas(lds + (b0 & (NBUF - 1)) * BUFB, kf, [](auto) {});
      kprefetch(lds + ((b0 + 1) & (NBUF - 1)) * BUFB, kpre);
      sm_mask(s0, b0);
      sm_max0(s0);
      sm_max1(s0);
      sm_ref1();
      sm_ref2();
      sm_ref3();
      alpha = 1.f;  // O is still zero: no factor to apply
      static_for<0, 16>([&](auto xc) { sm_exp(s0, xc); });
      sm_pack(pc0, pc1);
    }

    // ------------------------------------------------------------------
    // Iteration b.  Entry: blocks b, b+1 resident for every wave, b+2 in
    // flight; the own rows' P^T(b) in pc0/pc1 and their factor in alpha (O
    // is not yet brought to the reference of block b); the first KDEPTH score
    // fragments of block b+1 in kpre; the slot of block b+3 in idx_cur.
    // The buffers an iteration touches are distinct, and the body says so
    // with restrict pointers: that lets the compiler see that the
    // transposing reads of block b cannot alias the gather into block b+3,
    // so it does not wait for that gather before them.
    //   dmab: block b+3 (gather target; held block b-1, whose last reader
    //         finished before the barrier at the top)
    //   vbuf: block b (values)   kbuf: block b+1 (scores; stale if none)
    //   nbuf: block b+2 (first score fragments of the next iteration)
    // The P^T and factor regions carry data between waves and are not
    // restrict: the compiler would assume no other wave writes them and
    // reuse values loaded before a barrier.
    // ------------------------------------------------------------------
    auto body = [&](int b, auto mask_tag, lds_char* __restrict__ dmab,
                    const lds_char* __restrict__ vbuf, const lds_char* __restrict__ kbuf,
                    const lds_char* __restrict__ nbuf) {
      constexpr bool MASK = decltype(mask_tag)::value;
      // everyone is done with block b-1 and with P^T(b-1) (all LDS reads but
      // the KDEPTH score fragments read ahead have returned)
      barrier_after<waitcnt_imm(VM_ANY, KDEPTH)>();

      // ---- phase A ----
      // the own rows' P^T(b) and factors for everyone
      lds_st(pbuf + 2048 * wave + pofs, pc0);
      lds_st(pbuf + 2048 * wave + 1024 + pofs, pc1);
      if (hl == 0) lds_st(abuf + 16 * l32 + 4 * wave, alpha);
      // gather of block b+3 (past the end: a valid row into a free buffer),
      // then the slot of block b+4.  The gather's address is formed before
      // the next index load, so no wait can cover that load.
      const auto gsrc = gather_src(idx_cur);
      const int gbase = gather_base(dmab);
      const int idx_next = load_idx(b + 4);

      const lds_char* vb0 = vbuf + vofs0;
      const lds_char* vb1 = vbuf + vofs1;
      auto vread = [&](int fb, int k2) {  // value fragment of own block fb, column half k2
        const int off = 2048 * fb + 1024 * k2;
        const bf16x4_t lo = lds_read_tr(vb0 + off);
        const bf16x4_t hi = lds_read_tr(vb1 + off);
        return (bf16x8_t)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      auto pread = [&](int rg, int k2) {
        return lds_ld<bf16x8_t>(pbuf + 2048 * rg + 1024 * k2 + pofs);
      };
      bf16x8_t vf[2][FB];  // value fragments [k2][fb]
      bf16x8_t pf[2][RG];  // P^T fragments [k2][rg]
      f32x4_t af;          // factors of the lane's row in each row group

      bf16x8_t kf[KS];
#pragma unroll
      for (int k = 0; k < KDEPTH; ++k) kf[k] = kpre[k];
      f32x16_t sn = score_mfmas(kbuf, kf, [&](auto kc) {
        constexpr int k = decltype(kc)::value;
        if constexpr (k % 3 == 1 && k / 3 < LPW)
          gather_one(gbase, gsrc, std::integral_constant<int, k / 3>{});
        if constexpr (k == SYNC_STEP) {
          // P^T(b) and the factors are complete (all LDS traffic but the
          // KDEPTH score reads ahead has returned); block b+2 has landed (only
          // block b+3's gather may still run; the slot of block b+4 is loaded)
          barrier_after<waitcnt_imm(LPW, KDEPTH)>();
        }
        if constexpr (k == SYNC_STEP + 1) af = lds_ld<f32x4_t>(abuf + 16 * l32);
        if constexpr (k >= SYNC_STEP + 1 && k < SYNC_STEP + 1 + RG)
          pf[0][k - SYNC_STEP - 1] = pread(k - SYNC_STEP - 1, 0);
        if constexpr (k >= SYNC_STEP + 3 && k < SYNC_STEP + 5)
          vf[0][k - SYNC_STEP - 3] = vread(k - SYNC_STEP - 3, 0);
      });
      vf[0][2] = vread(2, 0);

      // rare: some row's reference moved with block b -- bring O along first
      if (__ballot(af[0] != 1.f || af[1] != 1.f || af[2] != 1.f || af[3] != 1.f) != 0) {
        value_drain();
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
          for (int fb = 0; fb < FB; ++fb) {
            f32x16_t x = o[rg][fb];
            in_agprs(x);
            x *= af[rg];
            in_agprs(x);
            o[rg][fb] = x;
          }
        asm volatile("s_nop 4" ::: "memory");
      }

      // ---- phase B: values of block b, softmax of block b+1 ----
      const lds_char* nb0 = nbuf + kofs0;
      const lds_char* nb1 = nbuf + kofs1;
      // step i: k2 = i >> 4, fb = (i >> 2) & 3, rg = i & 3
      static_for<0, 2 * FB * RG>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int k2 = i >> 4, fb = (i >> 2) & 3, rg = i & 3;
        // value fragments three blocks ahead, P^T of the second k-half
        if constexpr (rg == 1) {
          constexpr int nf = k2 * FB + fb + 3;  // flat index [k2][fb] of the fragment to read
          if constexpr (nf < 2 * FB) vf[nf / FB][nf % FB] = vread(nf % FB, nf / FB);
        }
        if constexpr (k2 == 0 && fb == 2) pf[1][rg] = pread(rg, 1);
        value_mfma(o[rg][fb], vf[k2][fb], pf[k2][rg]);
        // the softmax of block b+1, spread so that no step carries more
        // VALU work than one MFMA covers; the dependent stages of the new
        // reference sit two steps apart
        if constexpr (i == 0 && MASK) sm_mask(sn, b + 1);
        if constexpr (i == 1) sm_max0(sn);
        if constexpr (i == 2) sm_max1(sn);
        if constexpr (i == 3) sm_ref1();
        if constexpr (i == 5) sm_ref2();
        if constexpr (i == 7) sm_ref3();
        if constexpr (i >= 8 && i < 24) sm_exp(sn, std::integral_constant<int, i - 8>{});
        if constexpr (i >= 2 * FB * RG - KDEPTH) {
          constexpr int k = i - (2 * FB * RG - KDEPTH);
          kpre[k] = lds_ld<bf16x8_t>((k & 1 ? nb1 : nb0) + 2048 * (k >> 1));
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      sm_pack(pc0, pc1);
      idx_cur = idx_next;
      // the accumulators leave the iteration settled: whatever the compiler
      // places between iterations (or after the loop) may touch them
      value_drain();
    };
    auto step = [&](int b, auto mask_tag) {
      body(b, mask_tag, lds + ((b + 3) & (NBUF - 1)) * BUFB, lds + (b & (NBUF - 1)) * BUFB,
           lds + ((b + 1) & (NBUF - 1)) * BUFB, lds + ((b + 2) & (NBUF - 1)) * BUFB);
    };

    // Iterations whose next block lies wholly inside the prefix need no mask;
    // the others (and the last, whose next block is past the segment) do.
    using NoMask = std::integral_constant<bool, false>;
    using Mask = std::integral_constant<bool, true>;
    const int b_full = min(b_end, g.P / KB);
    {
      int b = b_begin;
      for (; b + 1 < b_full; ++b) step(b, NoMask{});
      for (; b < b_end; ++b) step(b, Mask{});
    }

    value_drain();
    // ---- segment statistics of every row, then the output ----
    // the own rows' m and l for everyone (lane l32's row of row group wave)
    const float l_own = l_run + other_half(l_run);
    if (hl == 0) {
      lds_st(sbuf + 16 * l32 + 4 * wave, m_run);
      lds_st(sbuf + 512 + 16 * l32 + 4 * wave, l_own);
    }
    // Every wave is done with the block buffers, and the gathers past the
    // segment's end have landed: the buffers serve as staging space below.
    barrier_after<waitcnt_imm(0, 0)>();
    const f32x4_t mrow = lds_ld<f32x4_t>(sbuf + 16 * l32);
    const f32x4_t lrow = lds_ld<f32x4_t>(sbuf + 512 + 16 * l32);
    // The accumulator holds, in lane (l32, hl), features 32 fb + 8 gq + 4 hl
    // .. +3 of this wave's 128 (fo = 128 wave) for tile row 32 rg + l32: a
    // store straight from it would touch 32 rows per instruction.  The wave
    // stages its slab [rows][128 features] in its own part of the block
    // buffers (rows padded by 16 bytes, so that the 16 rows of a write phase
    // fall on distinct banks) and writes whole row segments from there.
    // Within one wave LDS accesses execute in order: no waits between the
    // staging writes, the reads and the next pass's writes.
    const int fo = 128 * wave;
    auto row_live = [&](int trow) { return t * MT + trow < g.R; };
    if (slot < 0) {
      if (b_begin < b_end) {  // empty split segments leave the output alone
        // bf16 rows of 256 bytes, all 128 rows in one pass
        constexpr int STR = 256 + 16;
        lds_char* stg = lds + wave * (MT * STR);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          const float inv = 1.f / lrow[rg];
#pragma unroll
          for (int fb = 0; fb < FB; ++fb)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              bf16x4_t v4;
#pragma unroll
              for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(o[rg][fb][4 * gq + e] * inv);
              lds_st(stg + (32 * rg + l32) * STR + 2 * (32 * fb + 8 * gq + 4 * hl), v4);
            }
        }
        // 16 lanes per row, 4 rows per instruction
        __bf16* out = static_cast<__bf16*>(p.out) + ((size_t)g.q0 * p.H + t * MT) * DV + fo + 8 * (lane & 15);
#pragma unroll 8
        for (int i = 0; i < MT / 4; ++i) {
          const int trow = 4 * i + (lane >> 4);
          const bf16x8_t v = lds_ld<bf16x8_t>(stg + trow * STR + 16 * (lane & 15));
          if (row_live(trow)) *reinterpret_cast<bf16x8_t*>(out + (size_t)trow * DV) = v;
        }
        if (p.lse && wave == 0 && hl == 0) {
#pragma unroll
          for (int rg = 0; rg < RG; ++rg)
            if (row_live(32 * rg + l32))
              p.lse[(size_t)g.q0 * p.H + t * MT + 32 * rg + l32] = (mrow[rg] + log2f(lrow[rg])) * LN2;
        }
      }
      continue;
    }
    {
      // The partial, normalised: O / l of every row, a weighted mean of the
      // c_kv rows it saw, in fp16 after a power-of-two scale per row and
      // feature quarter that brings its largest magnitude into [2^14, 2^15)
      // (any finite c_kv fits, and small rows keep fp16's full precision),
      // then the rows' m and l and the four quarters' inverse scales in fp32.
      // Lane layout of the accumulator: store (rg, fb, gp) of wave w writes
      // 1 KB contiguously, lane l's 16 bytes holding features 128 w + 32 fb +
      // 16 gp + 4 (l >> 5) .. +3 and the same + 8 of tile row 32 rg +
      // (l & 31), at half offset (((w RG + rg) FB + fb) 2 + gp) 512 + 8 l.
      // Row groups without a live row are not stored (nothing reads them); a
      // row that saw no column (l = 0, m = -inf) stores zeros, and the merge
      // skips it.
      float* base = p.ws + slot * slot_floats_bf16(MT);
      float* stats = base + (size_t)MT * DV / 2;  // m [MT], l [MT], 1 / scale [4][MT]
      _Float16* ob = reinterpret_cast<_Float16*>(base) + (size_t)wave * (RG * FB * 2 * 512) + 8 * lane;
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        if (t * MT + 32 * rg >= g.R) continue;
        const float inv = lrow[rg] > 0.f ? 1.f / lrow[rg] : 0.f;
        float mx = 0.f;  // the row's largest |O| in this quarter (lanes l and l ^ 32)
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fabsf(o[rg][fb][e]));
        mx = fmaxf(mx, other_half(mx)) * inv;
        int ex = 0;
        (void)frexpf(mx, &ex);  // mx < 2^ex (ex = 0 for mx = 0)
        ex = min(max(ex, -100), 100);
        const float f = inv * ldexpf(1.f, 15 - ex);
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int gp = 0; gp < 2; ++gp) {
            const f32x16_t& x = o[rg][fb];
            f16x8_t v8;
#pragma unroll
            for (int e = 0; e < 8; ++e) v8[e] = (_Float16)(x[8 * gp + e] * f);
            *reinterpret_cast<f16x8_t*>(ob + ((rg * FB + fb) * 2 + gp) * 512) = v8;
          }
        if (hl == 0) stats[2 * MT + wave * MT + 32 * rg + l32] = ldexpf(1.f, ex - 15);
      }
      if (wave == 0 && hl == 0) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          stats[32 * rg + l32] = mrow[rg];
          stats[MT + 32 * rg + l32] = lrow[rg];
        }
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

}  // namespace

int launch_bf16(const Params& p, int grid, hipStream_t s) {
  if (p.num_slots * (long long)ROWB <= 0xffffffffLL)
    hipLaunchKernelGGL((attn_bf16_kernel<true>), dim3(grid, p.L), dim3(NWAVE * 64), 0, s, p);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<false>), dim3(grid, p.L), dim3(NWAVE * 64), 0, s, p);
  return check_launch("verify_attn(bf16)");
}

}  // namespace attn
}  // namespace ddtree
