// Forward partial attention for causal context parallelism on gfx950 (CDNA4).
//
// One kernel serves both ABI calls: a single ring step (cp = 1 over the given
// keys) and a virtual rank's whole ring with every K/V shard resident (steps
// t = 0..cp-1 read the shard of rank (rank - t) mod cp), the partials of all
// steps merged on the fly in registers.  That is the guide's attn(Q_i, K_j,
// V_j) followed by combine() (Accelerate concept guide, "So how does it
// work?"), with softmax written as an online (running max / running sum)
// recurrence so no score matrix is ever stored.
//
// Work decomposition
//   A bf16 workgroup of NW wave64s owns NW * 32 query rows of one query head
//   (32 rows a wave) and walks the ring's key tiles in step order; each K and
//   V^T tile copied into LDS serves all its waves.  Two waves share each SIMD:
//   NW = 8 is one workgroup per CU, NW = 4 two (chosen per launch by the
//   expected keys per row).  Key tiles never cross a rank's shard.  Before the walk the workgroup lists the tiles it needs,
//   each tagged, per wave, as skipped, "full" (no mask needed) or "partial"
//   (per-element mask q_lo <= k_pos <= q_pos), from the position bounds of the
//   tile and of the wave's rows.
//
// Matrix-core mapping (bf16: v_mfma_f32_32x32x16_bf16; fp32: 32x32x2 f32)
//   Scores are computed transposed, S^T = K Q^T, so the accumulator column -- a
//   lane modulo 32 -- is a query row: each lane holds 16 scores of its own row
//   per 32-key sub-tile and the row max / row sum need one cross-lane exchange
//   (lane ^ 32).  The K operand rows are loaded in a permuted key order (bits 2
//   and 3 of the row index swapped) so that each lane's 8 consecutive
//   accumulator registers hold 8 consecutive keys; those registers, converted to
//   bf16, are directly the B operand of O^T += V^T P^T, with no trip through
//   LDS.  V is staged transposed ([d][keys]) so the V^T operand is one 16-byte
//   LDS read.  The output accumulator O^T likewise keeps one query row per
//   lane, so the online-softmax rescale is one multiply per register.
//
// bf16 data movement
//   K, V^T and the key positions of the next tile are copied HBM -> LDS by
//   buffer loads with the LDS-direct bit (no staging registers, no VALU), into
//   one of two statically addressed buffers while the current tile is computed.
//   Each tile gets its own buffer descriptor whose record count ends at the
//   shard's last valid key row, so the rows past it read as zero.  LDS rows are
//   XOR-swizzled in 16-byte chunks so that the 16 lanes served together read 16
//   distinct bank groups.
#include <hip/hip_runtime.h>

#include <climits>
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace cpattn {
namespace fwdk {

using namespace dev;

constexpr int kRowsPerWave = 32;
// The fp32 kernel: 8 waves, one workgroup per CU.
constexpr int kF32Waves = 8;
constexpr int kF32Threads = kF32Waves * 64;
constexpr int kF32BlockM = kF32Waves * kRowsPerWave;
constexpr int kListCap = 1024;          // active key tiles listed per pass
static_assert(kPreListMaxTiles <= kListCap, "a precomputed list is one pass");
constexpr float kRescaleLog2 = 8.0f;    // keep a stale running max while scores stay within 2^8 of it

struct KParams {
  const char* q;
  const char* k;
  const char* v;
  const int* q_pos;
  const int* q_lo;          // may be null
  const int* k_pos;
  const int* kpos_pad;      // bf16: key positions per tile slot, padding = kInvalidKey
  const int4* bounds;       // per key tile {min pos, max pos, gap lo, gap hi}
  const int* order;         // may be null: query tiles in dispatch order (heaviest first)
  const unsigned* lists;    // may be null (4-wave launches only): per query tile, its listed key tiles
  const int* lcnt;          // with lists: their counts
  char* o;
  float* lse;
  long long q_sb, q_sh, q_ss;
  long long k_sb, k_sh, k_ss;
  long long v_sb, v_sh, v_ss;
  long long o_sb, o_sh, o_ss;
  int B, Hq, Hkv, sq, sk, cp, rank, R, tpr, n_qtiles, out_bf16;
  int merge_acc;            // 1: (o, lse) hold a partial result over other keys (fp32) to merge into
  float c2;                 // softmax scale * log2(e)
};

// Work item of this workgroup.  Workgroups are dealt round-robin over the 8
// XCDs; each XCD gets a contiguous range of logical ids so that the query heads
// sharing one K/V head (and the same key tiles) run on the same L2.  Within a
// range, query tiles run from the last (most keys under a causal mask) to the
// first, or in the order of p.order (document masks: the tiles that list the
// most key tiles first, so the longest workgroups do not start last).
struct Item {
  int b, h, kvh, qt;
};
__device__ __forceinline__ Item map_block(const KParams& p) {
  const int logical = xcd_logical_block();
  const int g = p.Hq / p.Hkv;
  const int hg = logical % g;
  int rest = logical / g;
  Item it;
  it.qt = p.order ? p.order[rest % p.n_qtiles] : p.n_qtiles - 1 - rest % p.n_qtiles;
  rest /= p.n_qtiles;
  it.kvh = rest % p.Hkv;
  it.b = rest / p.Hkv;
  it.h = it.kvh * g + hg;
  return it;
}

template <int DT>
__device__ __forceinline__ void store_out(const KParams& p, const Item& it, int row, int hi, float m_run,
                                          float l_tot, const f32x16* oacc) {
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  const long long li = ((long long)it.b * p.Hq + it.h) * p.sq + row;
  const float lse_new = empty ? -INFINITY : (m_run + log2f(l_tot)) * kLn2;
  const long long obase = (long long)it.b * p.o_sb + (long long)it.h * p.o_sh + (long long)row * p.o_ss;
  if (p.merge_acc) {
    // combine() with the partial already in (o, lse), which covers other keys:
    // L = M + ln(e^(l1 - M) + e^(l2 - M)), O = e^(l1 - L) O1 + e^(l2 - L) O2;
    // (0, -inf) on either side is the identity.  Both lanes of the row read
    // the old LSE in the same load, before either writes.
    const float l1 = p.lse[li];
    const float M = fmaxf(l1, lse_new);
    float L = -INFINITY, w1 = 0.f, w2 = 0.f;
    if (M != -INFINITY) {
      L = M + logf(expf(l1 - M) + expf(lse_new - M));
      w1 = expf(l1 - L);
      w2 = expf(lse_new - L) * inv;
    }
    if (hi == 0) p.lse[li] = L;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        f32x4* dst = reinterpret_cast<f32x4*>(p.o + (obase + 32 * t + 8 * rg + 4 * hi) * 4);
        const f32x4 old = *dst;
        f32x4 val;
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = w1 * old[e] + w2 * oacc[t][4 * rg + e];
        *dst = val;
      }
    return;
  }
  if (hi == 0) p.lse[li] = lse_new;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int dv = 32 * t + 8 * rg + 4 * hi;
      const f32x4 val = {oacc[t][4 * rg] * inv, oacc[t][4 * rg + 1] * inv, oacc[t][4 * rg + 2] * inv,
                         oacc[t][4 * rg + 3] * inv};
      if (p.out_bf16) {
        __bf16 bv[4] = {(__bf16)val[0], (__bf16)val[1], (__bf16)val[2], (__bf16)val[3]};
        *reinterpret_cast<u32x2*>(p.o + (obase + dv) * 2) = __builtin_bit_cast(u32x2, bv);
      } else {
        *reinterpret_cast<f32x4*>(p.o + (obase + dv) * 4) = val;
      }
    }
}

// store_out with the rows regrouped through LDS first (d = 128, bf16 kernel):
// the wave's 32 rows x 32-column slice t go through the wave's own 4.5 KB
// slot, after which lane l owns row 8i + l/8 of the wave and columns 32t +
// 4(l%8) .. +3, so that every global access covers 8 whole rows of the slice
// instead of 32 quarter rows.  The per-row factors move to those lanes by
// shuffles; the arithmetic is store_out's.  Every lane of the wave takes part.
template <int DT>
__device__ __forceinline__ void store_out_rows(const KParams& p, const Item& it, int row0, int row, int hi, bool valid,
                                               float m_run, float l_tot, const f32x16* oacc, lds_char* slot) {
  // LDS pointer casts exist in the device pass only.
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int STR = 144;  // bytes per staged row (128 + 16: no bank conflicts on the writes)
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  const long long li = ((long long)it.b * p.Hq + it.h) * p.sq + row;
  const float lse_new = empty ? -INFINITY : (m_run + log2f(l_tot)) * kLn2;
  float w1 = 0.f, w2 = inv;
  if (p.merge_acc) {
    const float l1 = valid ? p.lse[li] : -INFINITY;
    const float M = fmaxf(l1, lse_new);
    float L = -INFINITY;
    w2 = 0.f;
    if (M != -INFINITY) {
      L = M + logf(expf(l1 - M) + expf(lse_new - M));
      w1 = expf(l1 - L);
      w2 = expf(lse_new - L) * inv;
    }
    if (valid && hi == 0) p.lse[li] = L;
  } else if (valid && hi == 0) {
    p.lse[li] = lse_new;
  }
  const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int kr = ln >> 3, c4 = 4 * (ln & 7), r32 = ln & 31, h32 = ln >> 5;
  float rw1[4], rw2[4];
  bool rok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rw1[i] = __shfl(w1, 8 * i + kr);
    rw2[i] = __shfl(w2, 8 * i + kr);
    rok[i] = row0 + 8 * i + kr < p.sq;
  }
  f32x4 x[DT][4];
#pragma unroll
  for (int t = 0; t < DT; ++t) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const f32x4 v = {oacc[t][4 * rg], oacc[t][4 * rg + 1], oacc[t][4 * rg + 2], oacc[t][4 * rg + 3]};
      *reinterpret_cast<f32x4*>(slot + r32 * STR + (8 * rg + 4 * h32) * 4) = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) x[t][i] = *reinterpret_cast<const f32x4*>(slot + (8 * i + kr) * STR + c4 * 4);
  }
  const long long obase = (long long)it.b * p.o_sb + (long long)it.h * p.o_sh + (long long)(row0 + kr) * p.o_ss + c4;
  if (p.merge_acc) {
    f32x4* dst[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = reinterpret_cast<f32x4*>(p.o + (obase + (long long)(8 * i) * p.o_ss) * 4);
    f32x4 old[DT][4];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) old[t][i] = rok[i] ? dst[i][8 * t] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 val;
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = rw1[i] * old[t][i][e] + rw2[i] * x[t][i][e];
        if (rok[i]) dst[i][8 * t] = val;
      }
    return;
  }
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!rok[i]) continue;
      const f32x4 val = {x[t][i][0] * rw2[i], x[t][i][1] * rw2[i], x[t][i][2] * rw2[i], x[t][i][3] * rw2[i]};
      const long long at = obase + (long long)(8 * i) * p.o_ss + 32 * t;
      if (p.out_bf16) {
        __bf16 bv[4] = {(__bf16)val[0], (__bf16)val[1], (__bf16)val[2], (__bf16)val[3]};
        *reinterpret_cast<u32x2*>(p.o + at * 2) = __builtin_bit_cast(u32x2, bv);
      } else {
        *reinterpret_cast<f32x4*>(p.o + at * 4) = val;
      }
    }
#endif
}

// ============================================================================
// bf16 kernel
// ============================================================================
template <int D>
struct Bf16Cfg {
  static constexpr int BN = kTileKeysBf16;       // keys per tile
  static constexpr int ROW = D * 2;              // bytes per K (or row-major V) row in LDS
  static constexpr int CHR = D / 8;              // 16-byte chunks per such row
  static constexpr int TROW = BN * 2;            // bytes per V^T row in LDS (transposed layout)
  static constexpr int TCHR = BN / 8;            // 16-byte chunks per V^T row
  static constexpr int TILE = BN * ROW;          // bytes per K or V tile (either layout)
  static constexpr int NBLK = TILE / 1024;       // 1 KB copy blocks per tile
  static constexpr int QREG = D / 16;
  static constexpr int DT = D / 32;
};

// Copies 16 bytes per lane from buffer rs at byte offset voff + soff into LDS
// at lds + 16 * lane (one 1 KB block per wave), or 4 bytes per lane into
// lds + 4 * lane (copy_lds4).  Written as inline assembly so that the
// compiler neither tracks these copies nor inserts waits for them: every wait
// for them in this file is an explicit vmcnt (its alias tracking otherwise
// makes some LDS reads wait for copies issued just before them).  The block
// sets M0 (the LDS base), gives the load the one wait state an M0 write needs
// before it, and puts M0 back, so the compiler's M0 survives; it has no
// register results.
__device__ __forceinline__ void copy_lds16(__amdgpu_buffer_rsrc_t rs, int voff, int soff, unsigned lds) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(rs), "s"(soff)
      : "memory");
}
__device__ __forceinline__ void copy_lds4(__amdgpu_buffer_rsrc_t rs, int voff, unsigned lds) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(rs)
      : "memory");
}
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(size_t)(const __attribute__((address_space(3))) char*)p;
}

// NW waves of 32 query rows each; two waves share each SIMD (NW = 8: one
// workgroup per CU; NW = 4: two).  VT: V is read from the transposed copy the
// prep kernel writes into the workspace ([d][keys] tiles, one 16-byte LDS read
// per V^T operand); otherwise from V itself, row-major tiles read transposed
// by ds_read_b64_tr_b16 (two 8-byte reads per operand, no copy of V).
template <int D, int NW, bool VT, bool PRE = false>
__global__ __launch_bounds__(NW * 64, 8 / NW) void fwd_bf16_kernel(KParams p) {
  // The body uses device-only buffer-descriptor types; the host pass only needs
  // the launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  using C = Bf16Cfg<D>;
  constexpr int BPW = C::NBLK / NW;  // 1 KB blocks of a K or V tile per wave
  static_assert(BPW >= 1 && C::NBLK % NW == 0, "copy split");
  __shared__ __attribute__((aligned(1024))) char sK0[C::TILE];
  __shared__ __attribute__((aligned(1024))) char sK1[C::TILE];
  __shared__ __attribute__((aligned(1024))) char sV0[C::TILE];
  __shared__ __attribute__((aligned(1024))) char sV1[C::TILE];
  __shared__ __attribute__((aligned(16))) int sP0[C::BN];
  __shared__ __attribute__((aligned(16))) int sP1[C::BN];
  __shared__ int2 sList[kListCap];
  __shared__ int sCnt[NW];
  __shared__ int sWb[NW][6];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps tile-class branches scalar
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const Item it = map_block(p);
  const int row = it.qt * (NW * kRowsPerWave) + wave * kRowsPerWave + l32;
  const bool valid = row < p.sq;

  // Precomputed list: its first 64 entries are loaded before the queries, so
  // that the first copies need not wait for the query loads.
  int pre_cnt = 0;
  unsigned pre_g0 = 0;
  if constexpr (PRE) {
    pre_cnt = p.lcnt[it.qt];
    // Unconditional (clamped into this tile's list) so that the wait for it
    // need not cover the loads issued after it.
    const int ntot = p.cp * p.tpr;
    pre_g0 = p.lists[(size_t)it.qt * ntot + min(lane, ntot - 1)];
    __builtin_amdgcn_sched_barrier(0);
  }
  // ---- query operand (B of S^T = K Q^T) in registers ----------------------
  bf16x8 qreg[C::QREG];
  int qp, ql;
  if constexpr (PRE) {
    // Loads without branches or selects, so that the wait for the list
    // entries above covers only them: lanes of rows past the end compute on a
    // copy of the last row, every lane's row is its own, and only valid rows
    // are stored.
    const int rc = min(row, p.sq - 1);
    const char* qrow = p.q + ((long long)it.b * p.q_sb + (long long)it.h * p.q_sh + (long long)rc * p.q_ss) * 2;
#pragma unroll
    for (int kk = 0; kk < C::QREG; ++kk)
      qreg[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + (16 * kk + 8 * hi) * 2));
    qp = p.q_pos[rc];
    ql = p.q_lo[rc];
  } else {
    const char* qrow = p.q + ((long long)it.b * p.q_sb + (long long)it.h * p.q_sh + (long long)row * p.q_ss) * 2;
#pragma unroll
    for (int kk = 0; kk < C::QREG; ++kk) {
      const u32x4 raw = valid ? *reinterpret_cast<const u32x4*>(qrow + (16 * kk + 8 * hi) * 2) : u32x4{0, 0, 0, 0};
      qreg[kk] = __builtin_bit_cast(bf16x8, raw);
    }
    qp = valid ? p.q_pos[row] : -1;
    ql = valid ? (p.q_lo ? p.q_lo[row] : 0) : INT_MAX;
  }
  static_assert(!PRE || NW == 4, "precomputed lists: 4-wave launches");
  constexpr bool pre = PRE;
  if (!pre) {
    wave_row_bounds(wave, lane, valid, qp, ql, sWb);
    __syncthreads();
  }

  // ---- per-lane constant addresses ------------------------------------------
  // Copies: each wave fills blocks wave, wave + NW, ... of every K and V tile;
  // lane l of a block fills the block's 16-byte physical slot l, holding the
  // logical chunk the row's swizzle maps there.
  const long long k_row_bytes = p.k_ss * 2;
  const long long v_row_bytes = p.v_ss * 2;
  int voffK[BPW], voffV[BPW];
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    const int c = (wave + NW * j) * 64 + lane;  // physical 16-byte slot of the tile
    {
      const int r = c / C::CHR, ph = c % C::CHR;
      voffK[j] = (int)(r * k_row_bytes) + 16 * swz<C::CHR>(r, ph);
      if constexpr (!VT) voffV[j] = (int)(r * v_row_bytes) + 16 * swz_t<C::CHR>(r, ph);
    }
    if constexpr (VT) {
      const int r = c / C::TCHR, ph = c % C::TCHR;  // V^T: row d, chunk of 8 keys
      voffV[j] = (int)(r * v_row_bytes) + 16 * swz<C::TCHR>(r, ph);
    }
  }
  // K operand reads: rows key_perm(l32) (+32 for the second sub-tile), logical
  // chunk 2kk + hi of the row-swizzled K tile.
  const int krow = key_perm(l32);
  int kaddr[C::QREG];
#pragma unroll
  for (int kk = 0; kk < C::QREG; ++kk) kaddr[kk] = krow * C::ROW + 16 * swz<C::CHR>(krow, 2 * kk + hi);
  // V^T operand of key group kg (16 keys) and output tile t (32 columns of d):
  //  - VT: V^T row 32t + l32 (a column of d), chunk 2kg + hi (8 keys): one
  //    16-byte read at vaddr[kg] + t*32*TROW;
  //  - row-major: lane s16 of its 16-lane group reads key 16kg + 8hi + 4h +
  //    s16/4 at column 32t + 16*(bit 4 of lane) + 4*(s16%4) (h = 0, 1: two
  //    8-byte transposing reads), so the lane receives column 32t + l32 at
  //    keys 16kg + 8hi .. +7; byte offset xo[t] (+ xd for h = 1) + 16kg*ROW.
  int vaddr[VT ? 4 : 1], xo[VT ? 1 : C::DT], xd = 0;
  if constexpr (VT) {
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) vaddr[kg] = l32 * C::TROW + 16 * swz<C::TCHR>(l32, 2 * kg + hi);
  } else {
    const int s16 = lane & 15;
    const int cl = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1);
    int tP[2], tA = 0;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int r = 8 * hi + 4 * hh + (s16 >> 2);
      const int f = swz_t<C::CHR>(r, 0);
      tP[hh] = r * C::ROW + 16 * (cl ^ (f & 3)) + 8 * (s16 & 1);
      tA = 64 * (f >> 2);
    }
#pragma unroll
    for (int t = 0; t < C::DT; ++t) xo[t] = tP[0] + ((64 * t) ^ tA);
    xd = tP[1] - tP[0];
  }

  const char* kbase = p.k + ((long long)it.b * p.k_sb + (long long)it.kvh * p.k_sh) * 2;
  const char* vbase = p.v + ((long long)it.b * p.v_sb + (long long)it.kvh * p.v_sh) * 2;
  // V^T: one descriptor over this (batch, kv head)'s whole copy (d rows).
  const __amdgpu_buffer_rsrc_t rsVT =
      __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, VT ? (int)(D * v_row_bytes) : 0, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsP =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.kpos_pad, 0, 0x7fffffff, kBufferFlags);

  auto kbuf = [&](auto bc) -> char* { if constexpr (decltype(bc)::value) return sK1; else return sK0; };
  auto vbuf = [&](auto bc) -> char* { if constexpr (decltype(bc)::value) return sV1; else return sV0; };
  auto pbuf = [&](auto bc) -> int* { if constexpr (decltype(bc)::value) return sP1; else return sP0; };
  // A list entry, as this wave sees it: src | i << 8 for key tile i of rank
  // src's shard (tile id src * tpr + i), and the wave's class of the tile in
  // bits 24-25.
  auto rows_of = [&](unsigned e, int& r0, int& nval) {
    const int src = e & 0xFF, i = (e >> 8) & 0xFFFF;
    r0 = src * p.R + i * C::BN;
    nval = min(C::BN, p.R - i * C::BN);
  };
  auto tile_of = [&](unsigned e) { return (int)(e & 0xFF) * p.tpr + (int)((e >> 8) & 0xFFFF); };
  // Copy source of a tile's K (or V) rows: a descriptor whose record count
  // ends at the shard's last valid row, so rows past it read as zero, and a
  // byte offset.  A copy that is not needed (ok false) gets a descriptor of
  // no records: it writes zeros into the free buffer.
  struct Src {
    __amdgpu_buffer_rsrc_t rs;
    int soff;
  };
  auto k_src = [&](unsigned e, bool ok) {
    int r0, nval;
    rows_of(e, r0, nval);
    return Src{__builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (long long)r0 * k_row_bytes), 0,
                                                 ok ? (int)(nval * k_row_bytes) : 0, kBufferFlags),
               0};
  };
  // V, or V^T (the tile's 64 key columns, zero in the padding of a shard's
  // last tile).
  auto v_src = [&](unsigned e, bool ok) {
    if constexpr (VT) {
      return Src{ok ? rsVT : __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, 0, kBufferFlags),
                 tile_of(e) * C::BN * 2};
    } else {
      int r0, nval;
      rows_of(e, r0, nval);
      return Src{__builtin_amdgcn_make_buffer_rsrc((void*)(vbase + (long long)r0 * v_row_bytes), 0,
                                                   ok ? (int)(nval * v_row_bytes) : 0, kBufferFlags),
                 0};
    }
  };
  // This wave's share of a K or V tile copy: blocks wave, wave + NW, ...
  auto copy_k = [&](auto bc, const Src& sr, int j) {
    copy_lds16(sr.rs, voffK[j], sr.soff, lds_addr(kbuf(bc) + (wave + NW * j) * 1024));
  };
  auto copy_v = [&](auto bc, const Src& sr, int j) {
    copy_lds16(sr.rs, voffV[j], sr.soff, lds_addr(vbuf(bc) + (wave + NW * j) * 1024));
  };
  // The key positions of tile e (wave 0; padding slots kInvalidKey).
  auto copy_pos = [&](auto bc, unsigned e) {
    if (wave == 0) copy_lds4(rsP, tile_of(e) * C::BN * 4 + lane * 4, lds_addr(pbuf(bc)));
  };

  // ---- online softmax state ------------------------------------------------
  f32x16 oacc[C::DT];
#pragma unroll
  for (int t = 0; t < C::DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
  // Running max of scale*log2(e)*s (equal in lanes l and l^32) and this lane's
  // part of the running sum.  Exponentials of a tile are taken against the
  // running max as it stands; only when a lane's partial sum for the tile is
  // not finite or exceeds 2^40 (first tile of a row, or scores far above the
  // running max) is the tile's true max taken and the tile redone.
  float m_run = -INFINITY;
  float l_run = 0.f;
  constexpr float kRedo = 1099511627776.0f;  // 2^40
  bf16x8 pb[4];  // P^T of the current tile, bf16: the B operands of its P V MFMAs

  // S^T = K Q^T of the tile in K buffer kbc: 16 MFMAs into (s0, s1).
  auto scores = [&](auto kbc, f32x16& s0, f32x16& s1) {
    const char* sK = kbuf(kbc);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = 0.f;
      s1[r] = 0.f;
    }
#pragma unroll
    for (int kk = 0; kk < C::QREG; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + kaddr[kk]);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(sK + kaddr[kk] + 32 * C::ROW);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, qreg[kk], s1, 0, 0, 0);
    }
  };
  // P = exp2(c2*s - m) of group kg (8 keys) rounded to bf16; the fp32 values
  // go into the tile's row sum (the LSE needs them unrounded).
  auto expg = [&](const f32x16& c0, const f32x16& c1, int kg, float nm, bf16x8& pbk, float& lj) {
    const f32x16& sv = kg < 2 ? c0 : c1;
    const int base = 8 * (kg & 1);
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[base + j], p.c2, nm));
      const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[base + j + 1], p.c2, nm));
      const bf16x2 pr = __builtin_convertvector((f32x2){e0, e1}, bf16x2);
      lj += e0 + e1;
      pbk[j] = pr[0];
      pbk[j + 1] = pr[1];
    }
  };

  // One tile: its scores (c0, c1) are masked (key positions in buffer vbc),
  // exponentiated into pb while the next tile's scores are computed into (n0,
  // n1) from K buffer kbc, then multiplied into O with V from buffer vbc.
  // dk, dv: sources of the copies this tile's stage issues, K of the tile
  // after next into the K buffer other than kbc and V of the next tile into
  // the V buffer other than vbc, spread over the score chunks: issued
  // together, the copies of all waves queue at the vector memory unit and
  // stall the waves behind them.
  auto stage = [&](auto kbc, auto vbc, f32x16& c0, f32x16& c1, f32x16& n0, f32x16& n1, int cls_cur, const Src& dk,
                   const Src& dv) {
    using KO = std::integral_constant<int, 1 - decltype(kbc)::value>;
    using VO = std::integral_constant<int, 1 - decltype(vbc)::value>;
    const int* sP = pbuf(vbc);
    // Register r of sub-tile sub holds key 32*sub + 16*(r/8) + 8*hi + r%8.
    if (cls_cur == kPartial) {
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int* kp = sP + 16 * gg + 8 * hi;
        const int4 k0 = *reinterpret_cast<const int4*>(kp);
        const int4 k1 = *reinterpret_cast<const int4*>(kp + 4);
        const int kv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bool ok = kv[j] >= ql && kv[j] <= qp;
          if (gg < 2) c0[8 * gg + j] = ok ? c0[8 * gg + j] : -INFINITY;
          else c1[8 * (gg - 2) + j] = ok ? c1[8 * (gg - 2) + j] : -INFINITY;
        }
      }
    }
    // One straight-line block: the next tile's scores are computed even when
    // there is no next tile or this wave skips it, and this tile's
    // exponentials even when this wave skips it; such results go unused.
    float lj = 0.f;
    const float nm = -m_run;
    {
      // 16 chunks, fenced from each other: chunk m reads the K operand of MFMA
      // m+PF, issues MFMA m of the next tile's scores (sub-tile m%2, d-slice
      // m/2), and exponentiates scores 2m, 2m+1 of this tile.
      const char* sK = kbuf(kbc);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        n0[r] = 0.f;
        n1[r] = 0.f;
      }
      auto kop = [&](int m) {
        return *reinterpret_cast<const bf16x8*>(sK + kaddr[m >> 1] + (m & 1) * 32 * C::ROW);
      };
      // Issue priority 1 for this block, 0 again for the P V MFMAs: while one
      // wave interleaves scores and exponentials, the SIMD's other wave fills
      // the gaps.
      __builtin_amdgcn_s_setprio(1);
      constexpr int NM = 2 * C::QREG;  // MFMAs per tile
      constexpr int PF = 3;            // operand reads in flight
      bf16x8 ops[NM];
#pragma unroll
      for (int m = 0; m < PF; ++m) ops[m] = kop(m);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        constexpr int NC = 2 * BPW;                      // copy instructions per tile
        constexpr int STEP = NM / NC > 1 ? NM / NC : 1;  // chunks between them
        if (m % STEP == 0 && m / STEP < NC) {
          const int i = m / STEP;
          if (i < BPW) copy_k(KO{}, dk, i);
          else copy_v(VO{}, dv, i - BPW);
        }
        if (m + PF < NM) ops[m + PF] = kop(m + PF);
        if (m & 1) n1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ops[m], qreg[m >> 1], n1, 0, 0, 0);
        else n0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ops[m], qreg[m >> 1], n0, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < 32 / NM; q += 2) {
          const int x = (32 / NM) * m + q;  // score index: sub-tile x/16, register x%16
          const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x < 16 ? c0[x] : c1[x - 16], p.c2, nm));
          const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x < 16 ? c0[x + 1] : c1[x - 15], p.c2, nm));
          const bf16x2 pr = __builtin_convertvector((f32x2){e0, e1}, bf16x2);
          lj += e0 + e1;
          pb[x >> 3][x & 7] = pr[0];
          pb[x >> 3][(x & 7) + 1] = pr[1];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Pin the exponentials to this block: without a use here the compiler
    // sinks them past the skip test below, out of the interleave.
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) asm volatile("" : : "v"(__builtin_bit_cast(u32x4, pb[kg])));
    asm volatile("" : : "v"(lj));
    if (cls_cur == kSkip) return;
    // Redo against the tile's own max where a lane's sum is not finite or too
    // large; both lanes of a row take the same decision.
    const unsigned long long bal = __ballot(!(lj <= kRedo));
    const unsigned long long both = bal | (bal >> 32) | (bal << 32);
    if (both) {
      const bool mine = (both >> lane) & 1ull;
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(c0[r], c1[r]));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = mine ? fmaxf(m_run, mx * p.c2) : m_run;
      const float alpha = mnew == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - mnew);
      m_run = mnew;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < C::DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
      const float nm2 = m_run == -INFINITY ? 0.f : -m_run;
      lj = 0.f;
#pragma unroll
      for (int kg = 0; kg < 4; ++kg) expg(c0, c1, kg, nm2, pb[kg], lj);
    }
    l_run += lj;
    __builtin_amdgcn_s_setprio(0);
    // O^T += V^T P^T in 16 fenced chunks: chunk m reads the V^T operand of
    // MFMA m+PF (key group (m+PF)/DT, output tile (m+PF)%DT) and issues MFMA
    // m, so every MFMA finds its operand read PF MFMAs earlier (left to
    // itself the compiler reads each pair just before use, which exposes the
    // LDS latency on every pair).
    const char* sV = vbuf(vbc);
    constexpr int NMV = 4 * C::DT;  // P V MFMAs per tile
    constexpr int PFV = 3;
    auto vop = [&](int m) {
      const int kg = m / C::DT, t = m % C::DT;
      if constexpr (VT) {
        return *reinterpret_cast<const bf16x8*>(sV + vaddr[kg] + t * 32 * C::TROW);
      } else {
        const lds_char* g = to_lds(const_cast<char*>(sV)) + kg * 16 * C::ROW;
        return lds_read_tr(g + xo[t], g + (xo[t] + xd));
      }
    };
    bf16x8 va[NMV];
#pragma unroll
    for (int m = 0; m < PFV; ++m) va[m] = vop(m);
#pragma unroll
    for (int m = 0; m < NMV; ++m) {
      if (m + PFV < NMV) va[m + PFV] = vop(m + PFV);
      oacc[m % C::DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[m], pb[m / C::DT], oacc[m % C::DT], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- walk the ring: list the needed key tiles, then stream them ---------
  // Iteration j reads K of tile j+1 and V of tile j while tile j+2's K and
  // tile j+1's V (and key positions) are copied in; buffers alternate, so the
  // loop is unrolled by two with static buffer and register roles.  Each copy
  // has the iteration to land: every wave waits for its own copies at the end
  // of the iteration, before the barrier after which any wave reads them.
  f32x16 sa0, sa1, sb0, sb1;
  const int total = p.cp * p.tpr;
  const int csh = 2 * wave;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  for (int u0 = 0; u0 < total; u0 += kListCap) {
    const int cnt = pre ? pre_cnt
                        : build_key_list<C::BN, NW, kListCap>(p.bounds, p.tpr, p.R, p.rank, p.cp, u0,
                                                              min(total, u0 + kListCap), tid, wave, lane, sWb,
                                                              sList, sCnt);
    if (cnt == 0) continue;
    // Lane l of vl holds list slot lbase + l as this wave sees it (0 past the
    // end): an iteration takes its entry with v_readlane, not an LDS round trip.
    int lbase = 0;
    unsigned vl = 0;
    auto fill = [&](int b) {
      lbase = b;
      unsigned v = 0;
      if (b + lane < cnt) {
        if constexpr (PRE) {
          const unsigned g = p.lists[(size_t)it.qt * total + b + lane];
          v = (g & 0xFFFFFFu) | (((g >> (24 + csh)) & 3u) << 24);
        } else {
          const int2 e = sList[b + lane];
          v = (unsigned)e.x | ((((unsigned)e.y >> csh) & 3u) << 24);
        }
      }
      vl = v;
    };
    auto slot = [&](int j) { return (unsigned)__builtin_amdgcn_readlane((int)vl, j - lbase); };
    auto cls_of = [](unsigned e) { return (int)(e >> 24); };
    if constexpr (PRE) {
      lbase = 0;
      vl = lane < cnt ? (pre_g0 & 0xFFFFFFu) | (((pre_g0 >> (24 + csh)) & 3u) << 24) : 0u;
    } else {
      fill(0);
    }
    unsigned e_cur = slot(0), e_nxt = slot(1);
    copy_pos(I0{}, e_cur);
    {
      const Src k0 = k_src(e_cur, true), v0 = v_src(e_cur, true), k1 = k_src(e_nxt, cnt > 1);
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        copy_k(I0{}, k0, j);
        copy_v(I0{}, v0, j);
        copy_k(I1{}, k1, j);
      }
    }
    wait_vmem();
    __syncthreads();
    if (cls_of(e_cur) != kSkip) scores(I0{}, sa0, sa1);
    __syncthreads();
    for (int j = 0;;) {
      // K of tile j+1 in buffer 1, V of tile j in buffer 0; scores of tile j in sa.
      {
        if (j + 2 - lbase >= 64) fill(j + 2);
        const unsigned e2 = slot(j + 2);
        copy_pos(I1{}, e_nxt);
        stage(I1{}, I0{}, sa0, sa1, sb0, sb1, cls_of(e_cur), k_src(e2, j + 2 < cnt), v_src(e_nxt, j + 1 < cnt));
        wait_vmem();
        __syncthreads();
        e_cur = e_nxt;
        e_nxt = e2;
      }
      if (++j >= cnt) break;
      // K of tile j+1 in buffer 0, V of tile j in buffer 1; scores of tile j in sb.
      {
        if (j + 2 - lbase >= 64) fill(j + 2);
        const unsigned e2 = slot(j + 2);
        copy_pos(I0{}, e_nxt);
        stage(I0{}, I1{}, sb0, sb1, sa0, sa1, cls_of(e_cur), k_src(e2, j + 2 < cnt), v_src(e_nxt, j + 1 < cnt));
        wait_vmem();
        __syncthreads();
        e_cur = e_nxt;
        e_nxt = e2;
      }
      if (++j >= cnt) break;
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if constexpr (D == 128) {
    // The K/V tiles' space is read by no wave after the loop's last barrier:
    // three 4.5 KB slots per 16 KB buffer.
    static_assert(3 * 32 * 144 <= C::TILE && NW <= 9, "three output slots per tile buffer");
    wait_vmem();
    char* sb = wave < 3 ? sK0 : (wave < 6 ? sK1 : sV0);
    store_out_rows<C::DT>(p, it, it.qt * (NW * kRowsPerWave) + wave * kRowsPerWave, row, hi, valid, m_run, l_tot,
                          oacc, to_lds(sb) + (wave % 3) * 32 * 144);
  } else if (valid) {
    store_out<C::DT>(p, it, row, hi, m_run, l_tot, oacc);
  }
#endif
}

// ============================================================================
// fp32 kernel (exact-precision path: P stays fp32; staged through registers)
// ============================================================================
template <int D>
struct F32Cfg {
  static constexpr int BN = kTileKeysF32;        // 32 keys per tile
  static constexpr int KCHR = D / 4;             // 16-byte chunks per row
  static constexpr int CHUNKS = BN * KCHR;       // per tile, for K and for V
  static constexpr int LD = CHUNKS / kF32Threads;   // staged chunks per thread
  static constexpr int QREG = D / 2;
  static constexpr int DT = D / 32;
  static_assert(CHUNKS % kF32Threads == 0, "tile not divisible");
};

template <int D>
__global__ __launch_bounds__(kF32Threads, 1) void fwd_f32_kernel(KParams p) {
  using C = F32Cfg<D>;
  __shared__ __attribute__((aligned(16))) u32x4 sK[2][C::CHUNKS];
  __shared__ __attribute__((aligned(16))) u32x4 sV[2][C::CHUNKS];
  __shared__ __attribute__((aligned(16))) int sKpos[2][C::BN];
  __shared__ int2 sList[kListCap];
  __shared__ int sCnt[kF32Waves];
  __shared__ int sWb[kF32Waves][6];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const Item it = map_block(p);
  const int row = it.qt * kF32BlockM + wave * kRowsPerWave + l32;
  const bool valid = row < p.sq;

  // Lane half hi holds d indices hi*D/2 .. hi*D/2 + D/2 - 1 of its row.
  float qreg[C::QREG];
  {
    const char* qrow = p.q + ((long long)it.b * p.q_sb + (long long)it.h * p.q_sh + (long long)row * p.q_ss) * 4;
#pragma unroll
    for (int j = 0; j < D / 8; ++j) {
      const f32x4 raw = valid ? *reinterpret_cast<const f32x4*>(qrow + (hi * (D / 2) + 4 * j) * 4) : f32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) qreg[4 * j + e] = raw[e];
    }
  }
  const int qp = valid ? p.q_pos[row] : -1;
  const int ql = valid ? (p.q_lo ? p.q_lo[row] : 0) : INT_MAX;
  wave_row_bounds(wave, lane, valid, qp, ql, sWb);
  __syncthreads();

  f32x16 oacc[C::DT];
#pragma unroll
  for (int t = 0; t < C::DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  const long long kbase = (long long)it.b * p.k_sb + (long long)it.kvh * p.k_sh;
  const long long vbase = (long long)it.b * p.v_sb + (long long)it.kvh * p.v_sh;
  u32x4 kst[C::LD];
  u32x4 vst[C::LD];
  int kpst = kInvalidKey;

  auto stage_load = [&](int tile) {
    const int src = tile / p.tpr;
    const int i = tile - src * p.tpr;
    const int r0 = src * p.R + i * C::BN;
    const int nval = min(C::BN, p.R - i * C::BN);
#pragma unroll
    for (int j = 0; j < C::LD; ++j) {
      const int c = tid + j * kF32Threads;
      const int r = c / C::KCHR, ch = c % C::KCHR;
      kst[j] = r < nval ? *reinterpret_cast<const u32x4*>(p.k + ((kbase + (long long)(r0 + r) * p.k_ss) * 4 + ch * 16))
                        : u32x4{0, 0, 0, 0};
      vst[j] = r < nval ? *reinterpret_cast<const u32x4*>(p.v + ((vbase + (long long)(r0 + r) * p.v_ss) * 4 + ch * 16))
                        : u32x4{0, 0, 0, 0};
    }
    if (tid < C::BN) kpst = tid < nval ? p.k_pos[r0 + tid] : kInvalidKey;
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int j = 0; j < C::LD; ++j) {
      const int c = tid + j * kF32Threads;
      const int r = c / C::KCHR, ch = c % C::KCHR;
      sK[buf][r * C::KCHR + swz<C::KCHR>(r, ch)] = kst[j];
      sV[buf][c] = vst[j];
    }
    if (tid < C::BN) sKpos[buf][tid] = kpst;
  };

  auto compute = [&](int buf, int cls) {
    if (cls == kSkip) return;
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    const int kr = key_perm(l32);
#pragma unroll
    for (int j = 0; j < D / 8; ++j) {
      const f32x4 a = __builtin_bit_cast(f32x4, sK[buf][kr * C::KCHR + swz<C::KCHR>(kr, hi * (D / 8) + j)]);
#pragma unroll
      for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qreg[4 * j + e], s, 0, 0, 0);
    }
    if (cls == kPartial) {
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int* kp = &sKpos[buf][16 * gg + 8 * hi];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bool ok = kp[j] >= ql && kp[j] <= qp;
          s[8 * gg + j] = ok ? s[8 * gg + j] : -INFINITY;
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m_run, mx * p.c2);
    const bool need = mnew > m_run + kRescaleLog2;
    if (__any(need)) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mnew) : 1.f;
      m_run = need ? mnew : m_run;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < C::DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
    }
    const float nm = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], p.c2, nm));
      l_run += e;
      s[r] = e;
    }
    const float* vf = reinterpret_cast<const float*>(&sV[buf][0]);
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int key = 16 * (st >> 3) + 8 * hi + (st & 7);
#pragma unroll
      for (int t = 0; t < C::DT; ++t)
        oacc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf[key * D + 32 * t + l32], s[st], oacc[t], 0, 0, 0);
    }
  };

  const int total = p.cp * p.tpr;
  const int csh = 2 * wave;
  auto entry_tile = [&](int2 e) { return (e.x & 0xFF) * p.tpr + ((e.x >> 8) & 0xFFFF); };
  for (int u0 = 0; u0 < total; u0 += kListCap) {
    const int cnt = build_key_list<C::BN, kF32Waves, kListCap>(p.bounds, p.tpr, p.R, p.rank, p.cp, u0, min(total, u0 + kListCap), tid,
                                                  wave, lane, sWb, sList, sCnt);
    if (cnt == 0) continue;
    stage_load(entry_tile(sList[0]));
    stage_store(0);
    __syncthreads();
    for (int j = 0; j < cnt; ++j) {
      const int cur = j & 1;
      const bool has_next = j + 1 < cnt;
      const int e = __builtin_amdgcn_readfirstlane(sList[j].y);
      if (has_next) stage_load(entry_tile(sList[j + 1]));
      compute(cur, ((unsigned)e >> csh) & 3);
      if (has_next) stage_store(cur ^ 1);
      __syncthreads();
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (valid) store_out<C::DT>(p, it, row, hi, m_run, l_tot, oacc);
}

// Per key tile: position bounds {min pos, max pos, widest gap lo, gap hi}; for
// bf16 inputs also the key positions padded per tile slot (kInvalidKey in the
// padding of a shard's last tile), which the kernel copies into LDS with each
// tile for its per-element masks.  VT: also V transposed into the workspace
// ([b][kv head][d][tile * BN + key], zero in the padding of a shard's last
// tile), which the wide launch reads as V^T tiles.
template <bool BF16, int D, bool VT>
__global__ __launch_bounds__(256) void prep_kernel(const int* __restrict__ k_pos, const char* __restrict__ v,
                                                   long long v_sb, long long v_sh, long long v_ss, int Hkv,
                                                   int R, int tpr, int4* __restrict__ bounds,
                                                   int* __restrict__ kpos_pad, __bf16* vt, long long vt_row) {
  constexpr int BN = BF16 ? kTileKeysBf16 : kTileKeysF32;
  const int tile = blockIdx.x;
  const int src = tile / tpr;
  const int i = tile - src * tpr;
  const int r0 = src * R + i * BN;
  const int nval = min(BN, R - i * BN);
  const int tid = threadIdx.x;
  if (blockIdx.y == 0 && tid < 64) {
    const bool ok = tid < nval;
    const int kp = ok ? k_pos[r0 + tid] : 0;
    const int mn = wave_min(ok ? kp : INT_MAX);
    const int mx = wave_max(ok ? kp : INT_MIN);
    const int2 gp = largest_gap(wave_sort<64>(ok ? kp : INT_MAX, tid), nval, tid);
    if (tid == 0) bounds[tile] = int4{mn, mx, gp.x, gp.y};
    if (BF16 && tid < BN) kpos_pad[tile * BN + tid] = ok ? kp : kInvalidKey;
  }
  if constexpr (VT) {
    __shared__ __bf16 s[BN][D + 8];
    const int b = blockIdx.y / Hkv, kvh = blockIdx.y % Hkv;
    const char* vb = v + ((long long)b * v_sb + (long long)kvh * v_sh) * 2;
    constexpr int CH = D / 8;  // 16-byte chunks per V row
    for (int c = tid; c < BN * CH; c += 256) {
      const int r = c / CH, ch = c % CH;
      const u32x4 raw = r < nval ? *reinterpret_cast<const u32x4*>(vb + ((long long)(r0 + r) * v_ss + ch * 8) * 2)
                                 : u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(&s[r][ch * 8]) = raw;
    }
    __syncthreads();
    __bf16* out = vt + ((long long)blockIdx.y * D) * vt_row + (long long)tile * BN;
    for (int c = tid; c < D * (BN / 8); c += 256) {
      const int dv = c / (BN / 8), kc = c % (BN / 8);
      bf16x8 w;
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = s[kc * 8 + j][dv];
      *reinterpret_cast<bf16x8*>(out + (long long)dv * vt_row + kc * 8) = w;
    }
  }
}

// Dispatch order of a document-masked bf16 launch.  order_cost_kernel: per
// 128-row query tile (4 waves of 32 rows, as the launch deals them), the number
// of ring key tiles the tile's workgroup lists, by the forward's own rule
// (build_key_list); with lists, also the list itself (entry .x | .y << 24),
// which the 4-wave kernel then reads instead of building it in every
// workgroup.  order_sort_kernel: one workgroup sorts the tiles by that count,
// most first, ties by tile index, with a bitonic sort in LDS, and writes their
// indices to order.
// NW waves of 32 rows per query tile: 4 for the forward's launch, 8 for the
// backward's dQ kernel (whose key tiles have the same size and bounds).
template <int NW>
__global__ __launch_bounds__(NW * 64) void order_cost_kernel(const int* __restrict__ q_pos, const int* __restrict__ q_lo,
                                                             const int4* __restrict__ bounds, int sq, int R, int tpr,
                                                             int rank, int cp, int* __restrict__ cost,
                                                             unsigned* __restrict__ lists) {
  __shared__ int sWb[NW][6];
  __shared__ int sCnt[NW];
  __shared__ int2 sList[NW == 4 ? kPreListMaxTiles : 1];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int row = blockIdx.x * NW * kRowsPerWave + wave * kRowsPerWave + (lane & 31);
  const bool valid = row < sq;
  wave_row_bounds(wave, lane, valid, valid ? q_pos[row] : -1, valid ? q_lo[row] : INT_MAX, sWb);
  __syncthreads();
  const int total = cp * tpr;
  if constexpr (NW == 4) if (lists) {
    const int n = build_key_list<kTileKeysBf16, NW, kPreListMaxTiles>(bounds, tpr, R, rank, cp, 0, total, tid, wave,
                                                                     lane, sWb, sList, sCnt);
    unsigned* out = lists + (size_t)blockIdx.x * total;
    for (int i = tid; i < n; i += NW * 64) out[i] = (unsigned)sList[i].x | ((unsigned)sList[i].y << 24);
    if (tid == 0) cost[blockIdx.x] = n;
    return;
  }
  int cnt = 0;
  for (int u = tid; u < total; u += NW * 64) {
    const int t = u / tpr;
    const int i = u - t * tpr;
    int src = rank - t;
    if (src < 0) src += cp;
    const int4 bd = bounds[src * tpr + i];
    bool act = false;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      act |= bd.x <= sWb[w][1] && bd.y >= sWb[w][2] && !(bd.z < sWb[w][2] && sWb[w][1] < bd.w) &&
             !(sWb[w][4] < bd.x && bd.y < sWb[w][5]);
    cnt += act ? 1 : 0;
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) cnt += __shfl_xor(cnt, o);
  if (lane == 0) sCnt[wave] = cnt;
  __syncthreads();
  if (tid == 0) {
    int tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += sCnt[w];
    cost[blockIdx.x] = tot;
  }
}

__global__ __launch_bounds__(1024) void order_sort_kernel(const int* __restrict__ cost, int n, int* __restrict__ order) {
  __shared__ unsigned long long key[kOrderMaxTiles];
  int m = 1;
  while (m < n) m <<= 1;
  // key: count in the high word, ~index in the low word (distinct, so the
  // descending sort is total); padding 0 sorts last.
  for (int i = threadIdx.x; i < m; i += blockDim.x)
    key[i] = i < n ? ((unsigned long long)(unsigned)cost[i] << 32) | (0xFFFFFFFFu - (unsigned)i) : 0ull;
  __syncthreads();
  for (int k = 2; k <= m; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < m; i += blockDim.x) {
        const int l = i ^ j;
        if (l > i) {
          const unsigned long long a = key[i], b = key[l];
          const bool desc = (i & k) == 0;  // this block sorts descending
          if (desc ? a < b : a > b) {
            key[i] = b;
            key[l] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < n; i += blockDim.x) order[i] = (int)(0xFFFFFFFFu - (unsigned)key[i]);
}

template <bool BF16, int D>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  const FwdWorkspace w = fwd_workspace_layout(a.b, a.hkv, a.d, a.sq, a.sk, a.cp, a.in_dtype);
  char* ws = static_cast<char*>(a.ws);
  int4* bounds = reinterpret_cast<int4*>(ws + w.bounds_off);
  int* kpos_pad = reinterpret_cast<int*>(ws + w.kpos_off);
  __bf16* vt = reinterpret_cast<__bf16*>(ws + w.vt_off);
  // Launch shape of the bf16 kernel (the same result bits either way):
  //  - dense causal rings of >= 65536 keys (every row sees many keys): 8
  //    waves share each tile copy (one workgroup per CU), and V is read from
  //    a transposed copy (one 16-byte LDS read per V^T operand instead of two
  //    transposing reads; 2% faster at 131072 keys, prep pass included);
  //  - shorter rings and document masks (rows see fewer keys): two 4-wave
  //    workgroups per CU, whose barriers stay apart, reading V itself (no
  //    prep pass: 8-10% faster on the packed-document workloads).
  const bool wide = BF16 && a.q_lo == nullptr && fwd_wide_keys(a.in_dtype, a.sk);
  const bool use_vt = wide && !a.v_in_place;
  // Document masks make the work per query tile uneven: those launches
  // dispatch their query tiles heaviest first.
  const int n_order = (int)((a.sq + kOrderRows - 1) / kOrderRows);
  const bool ordered = BF16 && !wide && a.q_lo != nullptr && a.sk > 0 && n_order > 1 && n_order <= kOrderMaxTiles;
  int* order_cost = reinterpret_cast<int*>(ws + w.order_off);
  int* order = order_cost + n_order;
  const int ntiles = a.cp * a.tiles_per_rank;
  // Those of at most kPreListMaxTiles key tiles list each query tile's key
  // tiles once, here, for all heads (the same lists every workgroup of the
  // tile would build).
  const bool pre = ordered && a.pre_lists && ntiles <= kPreListMaxTiles;
  unsigned* lists = reinterpret_cast<unsigned*>(ws + w.list_off);
  if (ntiles > 0) {
    const dim3 grid(ntiles, use_vt ? a.b * a.hkv : 1);
    const long long vs[3] = {a.v_str[0], a.v_str[1], a.v_str[2]};
    if (use_vt)
      hipLaunchKernelGGL((prep_kernel<BF16, D, true>), grid, dim3(256), 0, stream, a.k_pos,
                         static_cast<const char*>(a.v), vs[0], vs[1], vs[2], a.hkv, a.rows_per_rank,
                         a.tiles_per_rank, bounds, kpos_pad, vt, (long long)w.vt_row);
    else
      hipLaunchKernelGGL((prep_kernel<BF16, D, false>), grid, dim3(256), 0, stream, a.k_pos,
                         static_cast<const char*>(a.v), vs[0], vs[1], vs[2], a.hkv, a.rows_per_rank,
                         a.tiles_per_rank, bounds, kpos_pad, vt, (long long)w.vt_row);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (ordered) {
    hipLaunchKernelGGL(order_cost_kernel<4>, dim3(n_order), dim3(256), 0, stream, a.q_pos, a.q_lo, bounds, (int)a.sq,
                       a.rows_per_rank, a.tiles_per_rank, a.rank, a.cp, order_cost, pre ? lists : nullptr);
    hipLaunchKernelGGL(order_sort_kernel, dim3(1), dim3(1024), 0, stream, order_cost, n_order, order);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  KParams p{};
  p.q = static_cast<const char*>(a.q);
  p.k = static_cast<const char*>(a.k);
  p.q_pos = a.q_pos;
  p.q_lo = a.q_lo;
  p.k_pos = a.k_pos;
  p.kpos_pad = kpos_pad;
  p.bounds = bounds;
  p.order = ordered ? order : nullptr;
  p.lists = pre ? lists : nullptr;
  p.lcnt = order_cost;
  p.o = static_cast<char*>(a.o);
  p.lse = a.lse;
  p.q_sb = a.q_str[0];
  p.q_sh = a.q_str[1];
  p.q_ss = a.q_str[2];
  p.k_sb = a.k_str[0];
  p.k_sh = a.k_str[1];
  p.k_ss = a.k_str[2];
  if (use_vt) {  // V^T copy: [b][hkv][d][vt_row]
    p.v = reinterpret_cast<const char*>(vt);
    p.v_ss = w.vt_row;
    p.v_sh = (long long)D * w.vt_row;
    p.v_sb = (long long)a.hkv * p.v_sh;
  } else {
    p.v = static_cast<const char*>(a.v);
    p.v_sb = a.v_str[0];
    p.v_sh = a.v_str[1];
    p.v_ss = a.v_str[2];
  }
  p.o_sb = a.o_str[0];
  p.o_sh = a.o_str[1];
  p.o_ss = a.o_str[2];
  p.B = a.b;
  p.Hq = a.hq;
  p.Hkv = a.hkv;
  p.sq = a.sq;
  p.sk = a.sk;
  p.cp = a.cp;
  p.rank = a.rank;
  p.R = a.rows_per_rank;
  p.tpr = a.tiles_per_rank;
  p.out_bf16 = a.out_dtype == CP_BF16;
  p.merge_acc = a.merge_acc;
  p.c2 = a.scale_log2;
  if constexpr (BF16) {
    const int nw = wide ? 8 : 4;
    p.n_qtiles = (a.sq + nw * kRowsPerWave - 1) / (nw * kRowsPerWave);
    const long long nblk = (long long)p.n_qtiles * a.hq * a.b;
    if (use_vt)
      hipLaunchKernelGGL((fwd_bf16_kernel<D, 8, true>), dim3((unsigned)nblk), dim3(8 * 64), 0, stream, p);
    else if (wide)
      hipLaunchKernelGGL((fwd_bf16_kernel<D, 8, false>), dim3((unsigned)nblk), dim3(8 * 64), 0, stream, p);
    else if (pre)
      hipLaunchKernelGGL((fwd_bf16_kernel<D, 4, false, true>), dim3((unsigned)nblk), dim3(4 * 64), 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<D, 4, false>), dim3((unsigned)nblk), dim3(4 * 64), 0, stream, p);
  } else {
    p.n_qtiles = (a.sq + kF32BlockM - 1) / kF32BlockM;
    const long long nblk = (long long)p.n_qtiles * a.hq * a.b;
    hipLaunchKernelGGL((fwd_f32_kernel<D>), dim3((unsigned)nblk), dim3(kF32Threads), 0, stream, p);
  }
  return hipGetLastError();
}

// Tile tables of the allocation-free forward (see fwd_noalloc_scratch).  In
// host code `scratch` names a host-side stand-in, not the device array: only
// the address hipGetSymbolAddress returns for the current device is ever used.
__device__ __attribute__((aligned(256))) char scratch[kNoAllocScratchBytes];

}  // namespace fwdk

hipError_t fwd_noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(fwdk::scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_order_sort(const int* cost, int n, int* order, hipStream_t stream) {
  hipLaunchKernelGGL(fwdk::order_sort_kernel, dim3(1), dim3(1024), 0, stream, cost, n, order);
  return hipGetLastError();
}

hipError_t launch_dq_order(const int* q_pos, const int* q_lo, const int4* kbounds, int sq, int R, int tpr, int rank,
                           int cp, int* cost, int* order, hipStream_t stream) {
  const int n = (sq + 255) / 256;
  hipLaunchKernelGGL(fwdk::order_cost_kernel<8>, dim3(n), dim3(512), 0, stream, q_pos, q_lo, kbounds, sq, R, tpr,
                     rank, cp, cost, nullptr);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  return launch_order_sort(cost, n, order, stream);
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  using namespace fwdk;
  if (a.in_dtype == CP_BF16) return a.d == 64 ? launch_t<true, 64>(a, stream) : launch_t<true, 128>(a, stream);
  return a.d == 64 ? launch_t<false, 64>(a, stream) : launch_t<false, 128>(a, stream);
}

}  // namespace cpattn
