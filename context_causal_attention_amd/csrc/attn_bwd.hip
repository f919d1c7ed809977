// Backward of causal context-parallel attention on gfx950 (CDNA4), recomputing
// the probabilities from the saved log-sum-exp: for every allowed (q, k) pair
//   P = exp(scale*q.k - LSE_q)          dV_k += P dO_q
//   dP = dO_q . v_k                      dS = P (dP - delta_q)
//   dQ_q += scale dS k_k                 dK_k += scale dS q_q
// with delta_q = dO_q . O_q.  Key/value heads sum over the query heads that read
// them.  On a real cluster the dK/dV partials of a ring step go back to the
// shard's owner; with every shard resident they accumulate in place.
//
// Two kernels, both without atomics (every output tile has one owner per call):
//   * dkdv_kernel: a workgroup owns 128 keys (32 a wave) of one K/V head and
//     streams the local query tiles (64 rows) of every query head of the group.
//     Scores are computed as S = Q K^T so that a lane owns one key: K and V of
//     the wave's keys are resident MFMA operands, and P and dS come out of the
//     accumulators already in the operand layout of dV^T += dO^T P and
//     dK^T += Q^T dS (query rows read in the permuted order of key_perm); the
//     dO^T and Q^T operands are read from the row-major tiles with transposing
//     LDS reads.
//   * dq_kernel: a workgroup owns 256 query rows (32 a wave) of one head and
//     walks the ring's key tiles like the forward; S^T = K Q^T, dP^T = V dO^T,
//     dQ^T += K^T dS^T, with Q and dO of the wave's rows resident.
// Operand tiles are copied HBM -> LDS by buffer loads with the LDS-direct bit;
// a small preparation pass tabulates tile bounds and per-row constants.
#include <hip/hip_runtime.h>

#include <climits>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace cpattn {
namespace bwdk {

using namespace dev;

constexpr int kQT = kBwdTile;  // query rows per streamed tile (dkdv) / per prep tile
constexpr int kKT = kBwdTile;  // keys per tile (dq) / per prep tile

struct BParams {
  const char* q;         // bf16 [b, hq, sq, d] (strides q_*)
  const char* k;         // bf16 [b, hkv, sk, d]
  const char* v;
  const char* dout;      // bf16, same layout as q
  const int* q_pos;
  const int* q_lo;       // may be null
  const int* k_pos;
  // workspace
  const int4* kbounds;   // per 64-key tile {min pos, max pos, gap lo, gap hi}
  const int* kpos_pad;   // per key slot, padding = kInvalidKey
  const int4* qbounds;   // per 64-row query tile {min pos, max pos, min lo, max lo}
  const int2* qholes;    // per query tile: widest hole in the union of its rows' [lo, pos]
  const int* qlo_pad;    // per query slot [sq_pad]: document start (padding INT_MIN)
  const int* qspan_pad;  // position - document start (padding 0)
  const float* nl2;      // [b][hq][sq_pad]: -LSE * log2(e), 0 in padding and where LSE = -inf
  const float* dlt;      // [b][hq][sq_pad]: -delta, 0 in padding
  const int* kv_order;   // may be null: the dK/dV kernel's key groups in dispatch order (most work first)
  const int* q_order;    // may be null: the dQ kernel's 256-row query tiles in dispatch order
  float* dq;             // fp32 [b, hq, sq, d] contiguous, accumulated
  float* dk;             // fp32 [b, hkv, sk, d] contiguous, accumulated
  float* dv;
  long long q_sb, q_sh, q_ss, k_sb, k_sh, k_ss, v_sb, v_sh, v_ss;
  int sq_pad;            // query rows per (b, head), padded to kQT
  int B, Hq, Hkv, sq, sk, cp, rank, R, tpr, nqt;
  float c2;              // scale * log2(e)
  float scale;
};

// ============================================================================
// Preparation
// ============================================================================
// Key side, per 64-key tile of a rank's shard: position bounds and padded key
// positions.
__global__ __launch_bounds__(64) void key_prep_kernel(BParams p, int4* __restrict__ kbounds,
                                                      int* __restrict__ kpos_pad) {
  const int tile = blockIdx.x;
  const int src = tile / p.tpr;
  const int i = tile - src * p.tpr;
  const int r0 = src * p.R + i * kKT;
  const int nval = min(kKT, p.R - i * kKT);
  const int tid = threadIdx.x;
  const bool ok = tid < nval;
  const int kp = ok ? p.k_pos[r0 + tid] : 0;
  const int mn = wave_min(ok ? kp : INT_MAX);
  const int mx = wave_max(ok ? kp : INT_MIN);
  const int2 gp = largest_gap(wave_sort<64>(ok ? kp : INT_MAX, tid), nval, tid);
  if (tid == 0) kbounds[tile] = int4{mn, mx, gp.x, gp.y};
  kpos_pad[tile * kKT + tid] = ok ? kp : kInvalidKey;
}

// Query side, per 64-row tile of one (batch, query head): -LSE in base 2 and
// delta padded to the tile grid; for the first (batch, head) also the tile's
// position bounds and each row's document start and span (position minus
// document start), the form the dK/dV kernel's mask test takes.
__global__ __launch_bounds__(64) void query_prep_kernel(BParams p, const float* __restrict__ lse,
                                                        const float* __restrict__ delta, int4* __restrict__ qbounds,
                                                        int2* __restrict__ qholes, int* __restrict__ qlo_pad,
                                                        int* __restrict__ qspan_pad, float* __restrict__ nl2,
                                                        float* __restrict__ dlt) {
  const int tile = blockIdx.x;
  const int r0 = tile * kQT;
  const int nval = min(kQT, p.sq - r0);
  const int tid = threadIdx.x;
  const int bh = blockIdx.y;  // b * Hq + h
  const bool ok = tid < nval;
  if (bh == 0) {
    const int qp = ok ? p.q_pos[r0 + tid] : -1;
    const int ql = ok ? (p.q_lo ? p.q_lo[r0 + tid] : 0) : INT_MAX;
    const int a = wave_min(ok ? qp : INT_MAX), b = wave_max(ok ? qp : INT_MIN);
    const int c = wave_min(ok ? ql : INT_MAX), d = wave_max(ok ? ql : INT_MIN);
    const int2 hole = interval_hole(ql, qp, ok, tid, nval);
    if (tid == 0) {
      qbounds[tile] = int4{a, b, c, d};
      qholes[tile] = hole;
    }
    qlo_pad[r0 + tid] = ok ? ql : INT_MIN;
    qspan_pad[r0 + tid] = ok ? (int)((unsigned)qp - (unsigned)ql) : 0;
  }
  const long long idx = (long long)bh * p.sq + r0 + tid;
  // A row without any allowed key (LSE = -inf) gets 0 rather than +inf: the
  // score kernels mask with a -inf score, and -inf * c + inf would be NaN.
  const float l = ok ? lse[idx] : 0.f;
  nl2[(long long)bh * p.sq_pad + r0 + tid] = (ok && l != -__builtin_inff()) ? -l * kLog2e : 0.f;
  dlt[(long long)bh * p.sq_pad + r0 + tid] = ok ? -delta[idx] : 0.f;
}

// delta_q = sum_d dO[q, d] * O[q, d] for rows q = (b*Hq + h)*sq + i (fewer
// than 2^31 rows, so row arithmetic is 32-bit).  32 lanes share a row, D/32
// consecutive elements a lane, so a half-wave reads a row's dO and O as one
// contiguous segment each; the 8 half-waves of a block take 8 consecutive
// rows a step, and kDeltaSteps steps with every load issued before the first
// product keep that many rows of loads in flight per thread.  One step: two
// or four, though up to 19% faster when the kernel runs alone, were 11%
// slower inside the backward step, where it follows the forward's output
// writes and the zeroing of dQ.
constexpr int kDeltaSteps = 1;
constexpr int kDeltaRowsPerBlock = 8 * kDeltaSteps;
template <int D, typename OT>
__global__ __launch_bounds__(256) void delta_kernel(const char* __restrict__ dout, long long do_sb, long long do_sh,
                                                    long long do_ss, const OT* __restrict__ o, long long o_sb,
                                                    long long o_sh, long long o_ss, float* __restrict__ delta, int Hq,
                                                    int sq, long long rows) {
  constexpr int PER = D / 32;  // elements per lane
  typedef __bf16 bfv __attribute__((__vector_size__(PER * sizeof(__bf16))));
  typedef OT ov_t __attribute__((__vector_size__(PER * sizeof(OT))));
  const int lane = threadIdx.x & 31;
  const unsigned r0 = blockIdx.x * (unsigned)kDeltaRowsPerBlock + (threadIdx.x >> 5);
  bfv dv[kDeltaSteps];
  ov_t ov[kDeltaSteps];
#pragma unroll
  for (int u = 0; u < kDeltaSteps; ++u) {
    const unsigned r = r0 + 8u * u;
    if (r < rows) {
      const unsigned bh = r / (unsigned)sq, i = r - bh * (unsigned)sq;
      const unsigned b = bh / (unsigned)Hq, h = bh - b * (unsigned)Hq;
      const __bf16* dp = reinterpret_cast<const __bf16*>(dout) + (long long)b * do_sb + (long long)h * do_sh +
                         (long long)i * do_ss + lane * PER;
      const OT* op = o + (long long)b * o_sb + (long long)h * o_sh + (long long)i * o_ss + lane * PER;
      dv[u] = *reinterpret_cast<const bfv*>(dp);
      ov[u] = *reinterpret_cast<const ov_t*>(op);
    } else {
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        dv[u][e] = (__bf16)0.f;
        ov[u][e] = (OT)0.f;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kDeltaSteps; ++u) {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc += (float)dv[u][e] * (float)ov[u][e];
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 32);
    const unsigned r = r0 + 8u * u;
    if (r < rows && lane == 0) delta[r] = acc;
  }
}

// ============================================================================
// dK, dV
// ============================================================================
// A workgroup of 8 waves owns 256 keys (32 a wave) of one K/V head and streams
// 64-row query tiles of the group's query heads through two LDS buffers.  Per
// 32-row half tile a wave computes S = Q K^T and dP = dO V^T (its keys as the
// MFMA columns: K from registers, V from LDS), then P and dS, then
// dV^T += dO^T P and dK^T += Q^T dS.  Two waves share each SIMD, so one wave's
// exponentials run while the other's MFMAs do, and LDS reads of two waves
// are in flight at once.
//
// Q and dO tiles are row-major in LDS with 16-byte chunks permuted per row by
// swz_t: one LDS-direct DMA instruction writes 4 (d = 128) or 8 (d = 64)
// whole rows, read from global memory as contiguous row segments, and both the
// row reads and the transposed reads are free of bank conflicts; a read's
// address is a lane pointer plus (lane constant XOR a per-read constant).
// The workgroup's V rows, copied once, use a column layout instead: chunk c of
// row r at c * col + 16 r, columns 64 bytes apart modulo 256, so 16 rows of
// one chunk are 256 contiguous bytes and every address is a lane pointer plus
// an immediate.
constexpr int kColBytes = kQT * 16 + 64;  // a column of a 64-row tile
constexpr int kKeysPerWg = 256;
static_assert(kKeysPerWg == 256, "bwd_kv_groups counts 256-key groups");
constexpr int kKvOrderDenseGroups = 256;  // dense rings of at most this many key groups are sorted too
constexpr int kVColBytes = kKeysPerWg * 16 + 64;

template <int D>
struct KvCfg {
  static constexpr int NW = 8;
  static constexpr int CHR = D / 8;              // 16-byte chunks per row
  static constexpr int ROW = D * 2;              // bytes per Q / dO row
  static constexpr int TILE = kQT * ROW;         // one Q or dO tile (row-major)
  static constexpr int NBLK = TILE / 1024;       // 1 KB DMA blocks per tile
  static constexpr int RPB = 1024 / ROW;         // rows per DMA block
  static constexpr int VTILE = CHR * kVColBytes; // the workgroup's V rows
  static constexpr int KREG = D / 16;            // 16-wide d slices
  static constexpr int DT = D / 32;              // 32-row blocks of dK^T / dV^T
  static constexpr int LIST = 1024;
  static_assert(CHR % NW == 0 || NW % CHR == 0, "column split");
  // The swizzle depends on row % 16; a wave's DMA blocks must all see the same
  // pattern so that one lane offset serves all of them.
  static_assert(NW % (16 / RPB) == 0 && NBLK % (16 / RPB) == 0 && (2 * NBLK) % NW == 0, "DMA split");
};

// Bounds of one wave's 32 keys (lanes l and l + 32 hold the same key):
// sKb[wave] = {min key pos, max key pos, all 32 keys valid, gap lo, gap hi},
// the gap being the widest between consecutive key positions.
__device__ __forceinline__ void kv_wave_bounds(bool kvalid, int kp, int wave, int lane, int (*sKb)[5]) {
  const int a = wave_min(kvalid ? kp : INT_MAX);
  const int c = wave_max(kvalid ? kp : INT_MIN);
  const bool all_valid = __all(kvalid);
  const int nk = __popcll(__ballot(kvalid) & 0xffffffffull);
  const int2 gp = largest_gap(wave_sort<32>(kvalid ? kp : INT_MAX, lane), nk, lane);
  if (lane == 0) {
    sKb[wave][0] = a;
    sKb[wave][1] = c;
    sKb[wave][2] = all_valid ? 1 : 0;
    sKb[wave][3] = gp.x;
    sKb[wave][4] = gp.y;
  }
}

// Class of 64-row query tile (bounds qb = {min pos, max pos, min lo, max lo},
// hole qh) for wave w's keys: skip when no key of the wave can lie in [min lo,
// max pos] of the tile (from the wave's key bounds and its largest gap between
// consecutive key positions, and the tile's widest hole), full when every key
// lies in [max lo, min pos] and the tile is whole.
__device__ __forceinline__ int kv_class(const int (*sKb)[5], int w, const int4& qb, const int2& qh, bool tile_full) {
  const int kmn = sKb[w][0], kmx = sKb[w][1];
  if (kmn != INT_MAX && kmn <= qb.y && kmx >= qb.z && !(sKb[w][3] < qb.z && qb.y < sKb[w][4]) &&
      !(qh.x < kmn && kmx < qh.y))
    return (sKb[w][2] && tile_full && kmx <= qb.x && kmn >= qb.w) ? kFull : kPartial;
  return kSkip;
}

// Dispatch cost of each 256-key group of the ring (8 waves of 32 keys, as the
// dK/dV kernel deals them): the number of 64-row query tiles some wave of the
// group needs (the same for every query head and kv head), by the kernel's
// own rule.
__global__ __launch_bounds__(512) void kv_cost_kernel(BParams p, int* __restrict__ cost) {
  constexpr int NW = 8;
  __shared__ int sKb[NW][5];
  __shared__ int sCnt[NW];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int tg = (p.R + kKeysPerWg - 1) / kKeysPerWg;
  const int src = blockIdx.x / tg;
  const int ig = blockIdx.x - src * tg;
  const int key0 = src * p.R + ig * kKeysPerWg;
  const int nkeys = min(kKeysPerWg, p.R - ig * kKeysPerWg);
  const int kloc = wave * 32 + (lane & 31);
  const bool kvalid = kloc < nkeys;
  kv_wave_bounds(kvalid, kvalid ? p.k_pos[key0 + kloc] : kInvalidKey, wave, lane, sKb);
  __syncthreads();
  int cnt = 0;
  for (int t = tid; t < p.nqt; t += NW * 64) {
    const int4 qb = p.qbounds[t];
    const int2 qh = p.qholes[t];
    bool act = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) act |= kv_class(sKb, w, qb, qh, false) != kSkip;
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

template <int D>
__global__ __launch_bounds__(512, 1) void dkdv_kernel(BParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = KvCfg<D>;
  constexpr int NW = C::NW;
  // Two buffers per tile kind, as separate arrays with roles fixed at compile
  // time: the compiler can then tell a tile's LDS reads from the DMA writes
  // into the other buffer, and does not wait for the copy in flight before
  // reading.
  __shared__ __attribute__((aligned(1024))) char sQ0[C::TILE];
  __shared__ __attribute__((aligned(1024))) char sQ1[C::TILE];
  __shared__ __attribute__((aligned(1024))) char sO0[C::TILE];
  __shared__ __attribute__((aligned(1024))) char sO1[C::TILE];
  // The smaller alignment places V after the four tiles, which then lie in the
  // first 64 KiB, where a tile read's constant part fits the DS offset field.
  __shared__ __attribute__((aligned(16))) char sV[C::VTILE];
  // Per row of each buffered tile: -LSE*log2(e), -delta, document start, span.
  __shared__ __attribute__((aligned(16))) float sR0[4][kQT];
  __shared__ __attribute__((aligned(16))) float sR1[4][kQT];
  __shared__ int2 sList[C::LIST];
  __shared__ int sCnt[NW];
  __shared__ int sKb[NW][5];  // per wave: min key pos, max key pos, all keys valid, gap lo, gap hi

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int s16 = lane & 15;
  const int g = p.Hq / p.Hkv;

  // ---- work item: 256 keys of rank src's shard, for one (batch, kv head) ----
  const int tg = (p.R + kKeysPerWg - 1) / kKeysPerWg;
  int logical = xcd_logical_block();
  const int gl = logical % (p.cp * tg);
  const int grp = p.kv_order ? p.kv_order[gl] : gl;
  logical /= p.cp * tg;
  const int kvh = logical % p.Hkv;
  const int b = logical / p.Hkv;
  const int src = grp / tg;
  const int ig = grp - src * tg;
  const int key0 = src * p.R + ig * kKeysPerWg;         // first key row of the workgroup in k_all
  const int nkeys = min(kKeysPerWg, p.R - ig * kKeysPerWg);
  const int kloc = wave * 32 + l32;
  const bool kvalid = kloc < nkeys;
  const int krow = key0 + kloc;
  const int kp = kvalid ? p.k_pos[krow] : kInvalidKey;

  // V rows of the workgroup into LDS (64 keys x one chunk per DMA instruction);
  // rows past the shard read as zero.
  {
    const long long v_row_bytes = p.v_ss * 2;
    const char* vb = p.v + ((long long)b * p.v_sb + (long long)kvh * p.v_sh + (long long)key0 * p.v_ss) * 2;
    const __amdgpu_buffer_rsrc_t rsV =
        __builtin_amdgcn_make_buffer_rsrc((void*)vb, 0, (int)(nkeys * v_row_bytes), kBufferFlags);
    constexpr int NI = C::CHR * (kKeysPerWg / 64);  // DMA instructions for V
#pragma unroll
    for (int j = 0; j < NI / NW; ++j) {
      const int i = wave + NW * j;
      const int col = i / (kKeysPerWg / 64), part = i % (kKeysPerWg / 64);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsV, (lds_ptr_t)(sV + col * kVColBytes + part * 1024), 16,
                                               (int)((part * 64 + lane) * v_row_bytes), col * 16, 0, 0);
    }
  }

  // K of this lane's key as the B operand of S (k-slots: d = 16kk + 8hi + j).
  bf16x8 kreg[C::KREG];
  {
    const char* kr = p.k + ((long long)b * p.k_sb + (long long)kvh * p.k_sh + (long long)krow * p.k_ss) * 2;
#pragma unroll
    for (int kk = 0; kk < C::KREG; ++kk)
      kreg[kk] = __builtin_bit_cast(bf16x8, kvalid ? *reinterpret_cast<const u32x4*>(kr + (16 * kk + 8 * hi) * 2)
                                                   : u32x4{0, 0, 0, 0});
  }
  kv_wave_bounds(kvalid, kp, wave, lane, sKb);
  __syncthreads();  // the list builder reads every wave's key bounds

  // ---- per-lane constant offsets ----------------------------------------
  const long long q_row_bytes = p.q_ss * 2;
  // DMA: blocks wave, wave + NW, ... of the Q and dO tiles; lane l fills slot
  // l % CHR of row l / CHR of its block.
  const int voff = (int)((lane / C::CHR) * q_row_bytes) +
                   16 * swz_t<C::CHR>(C::RPB * (wave % C::NBLK) + lane / C::CHR, lane % C::CHR);
  // Row reads (A of S = Q K^T and dP = dO V^T): row key_perm(l32) (+32 sub),
  // logical chunk 2kk + hi, at byte nrow*ROW + ((32 kk) ^ nY) of the tile.
  const int nrow = key_perm(l32);
  const int nY = 16 * (hi ^ swz_t<C::CHR>(nrow, 0));
  // V operand (B of dP): this lane's key at chunk 2kk + hi.
  const int vbase = hi * kVColBytes + kloc * 16;
  // Transposed reads (A of dV^T += dO^T P, dK^T += Q^T dS): lane s16 of its
  // 16-lane group reads row 8hi + 4h + s16/4 (+16gg + 32sub) at column 32t +
  // 16*(bit 4 of lane) + 4*(s16%4); the lane then holds column 32t + l32 at
  // rows 8hi + 4h + 0..3.  With the row's swizzle f, the logical chunk 4t + cl
  // lands at 4 (t ^ (f >> 2)) + (cl ^ (f & 3)): byte tP[h] + ((64 t) ^ tA).
  int tP[2], tA;
  {
    const int cl = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 8 * hi + 4 * h + (s16 >> 2);
      const int f = swz_t<C::CHR>(r, 0);
      tP[h] = r * C::ROW + 16 * (cl ^ (f & 3)) + 8 * (s16 & 1);
      tA = 64 * (f >> 2);  // the same for both h
    }
  }
  // A row read of the loop is a per-lane offset yo[kk] plus a constant
  // (buffer address, half-tile and dO offsets) that the DS offset field holds;
  // a transposed read of chunk group t uses xo[t] (+ xd for the second row
  // group) the same way.  These offsets pass
  // through an empty asm, in place, at the start of each half tile, so that
  // the compiler does not hoist offset + constant out of the loop as one
  // register per read.  V and the per-row arrays lie above 64 KiB: their
  // offsets carry the expected array address, which a constant in the read
  // subtracts again (another placement only costs an add per read).
  int yo[C::KREG];   // row reads: nrow*ROW + ((32 kk) ^ nY)
#pragma unroll
  for (int kk = 0; kk < C::KREG; ++kk) yo[kk] = nrow * C::ROW + ((32 * kk) ^ nY);
  // Transposed-read offsets of chunk group t for row group h = 0, and the
  // lane's distance to row group h = 1.
  int xo[C::DT];
#pragma unroll
  for (int t = 0; t < C::DT; ++t) xo[t] = tP[0] + ((64 * t) ^ tA);
  int xd = tP[1] - tP[0];
  constexpr int kVAt = 4 * C::TILE;            // expected address of sV
  constexpr int kRAt = 4 * C::TILE + C::VTILE;  // expected address of sR0
  int vo = vbase + kVAt;
  int ro8 = 32 * hi + kRAt;  // rows 8hi.. of the per-row arrays
  auto refresh = [&]() {
#pragma unroll
    for (int kk = 0; kk < C::KREG; ++kk) asm volatile("" : "+v"(yo[kk]));
#pragma unroll
    for (int t = 0; t < C::DT; ++t) asm volatile("" : "+v"(xo[t]));
    asm volatile("" : "+v"(xd), "+v"(vo), "+v"(ro8));
  };

  // ---- list of (query head, query tile) pairs this workgroup needs ---------
  // Entry .x = t | hg << 16 for tile t of query head kvh*g + hg; .y = class of
  // wave w << 2w: skip when no key of the wave can lie in [min lo, max pos] of
  // the tile (from the wave's key bounds and its largest gap between
  // consecutive key positions), full when every key lies in [max lo, min pos]
  // and the tile is whole.
  auto build = [&](int u0, int u1) {
    int cnt = 0;
    for (int base = u0; base < u1; base += NW * 64) {
      const int u = base + tid;
      bool act = false;
      int2 entry = {0, 0};
      if (u < u1) {
        const int hg = u / p.nqt;
        const int t = u - hg * p.nqt;
        const int4 qb = p.qbounds[t];
        const int2 qh = p.qholes[t];
        const bool tile_full = (t + 1) * kQT <= p.sq;
        entry.x = t | (hg << 16);
        unsigned bits = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const int cls = kv_class(sKb, w, qb, qh, tile_full);
          bits |= (unsigned)cls << (2 * w);
          act |= cls != kSkip;
        }
        entry.y = (int)bits;
      }
      const unsigned long long bal = __ballot(act);
      const int before = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) sCnt[wave] = __popcll(bal);
      __syncthreads();
      int off = cnt, tot = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        off += w < wave ? sCnt[w] : 0;
        tot += sCnt[w];
      }
      if (act) sList[off + before] = entry;
      cnt += tot;
      __syncthreads();
    }
    return cnt;
  };

  // ---- accumulators: dV^T and dK^T (row = d, column = this lane's key) -----
  f32x16 dva[C::DT], dka[C::DT];
#pragma unroll
  for (int t = 0; t < C::DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dva[t][r] = 0.f;
      dka[t][r] = 0.f;
    }

  // Buffers of compile-time index B.
  auto qbuf = [&](auto bc) -> char* { if constexpr (decltype(bc)::value) return sQ1; else return sQ0; };
  auto obuf = [&](auto bc) -> char* { if constexpr (decltype(bc)::value) return sO1; else return sO0; };
  auto rbuf = [&](auto bc) -> float* { if constexpr (decltype(bc)::value) return &sR1[0][0]; else return &sR0[0][0]; };

  // Copies query tile ex (t | hg << 16) into buffer B: the blocks of the Q and
  // dO tiles split over the waves; waves 0..3 each copy one per-row array.
  auto issue = [&](auto bc, int ex) {
    const int t = ex & 0xFFFF, hg = ex >> 16;
    const int h = kvh * g + hg;
    const int r0 = t * kQT;
    const int nval = min(kQT, p.sq - r0);
    const long long bh = (long long)b * p.Hq + h;
    const long long qoff = ((long long)b * p.q_sb + (long long)h * p.q_sh + (long long)r0 * p.q_ss) * 2;
    const __amdgpu_buffer_rsrc_t rsQ =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.q + qoff), 0, (int)(nval * q_row_bytes), kBufferFlags);
    const __amdgpu_buffer_rsrc_t rsO =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.dout + qoff), 0, (int)(nval * q_row_bytes), kBufferFlags);
    // 2*NBLK block copies (Q then dO) over NW waves.
#pragma unroll
    for (int j = 0; j < (2 * C::NBLK) / NW; ++j) {
      const int i = wave + NW * j;
      const int ib = i % C::NBLK;
      const int soff = (int)(C::RPB * ib * q_row_bytes);
      if (i < C::NBLK)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsQ, (lds_ptr_t)(qbuf(bc) + ib * 1024), 16, voff, soff, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsO, (lds_ptr_t)(obuf(bc) + ib * 1024), 16, voff, soff, 0, 0);
    }
    if (wave < 4) {
      const void* arr = wave == 0 ? (const void*)p.nl2 : wave == 1 ? (const void*)p.dlt
                      : wave == 2 ? (const void*)p.qlo_pad : (const void*)p.qspan_pad;
      const int soff = (int)((wave < 2 ? bh * p.sq_pad + r0 : (long long)r0) * 4);
      const __amdgpu_buffer_rsrc_t rsR = __builtin_amdgcn_make_buffer_rsrc((void*)arr, 0, 0x7fffffff, kBufferFlags);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsR, (lds_ptr_t)(rbuf(bc) + wave * kQT), 4, lane * 4, soff, 0, 0);
    }
  };

  // One half tile (sub) of the tile in buffer buf: S/dP, P/dS, dV/dK.
  auto half = [&](auto bc, int sub, bool full) {
    refresh();
    const lds_char* qn = to_lds(qbuf(bc)) + sub * 32 * C::ROW;
    const lds_char* on = to_lds(obuf(bc)) + sub * 32 * C::ROW;
    const lds_char* vn = to_lds(sV) + (vo - kVAt);
    const lds_char* rowb = to_lds(rbuf(bc)) + (ro8 - kRAt) + 32 * sub * 4;
    // S = Q K^T, dP = dO V^T: register r is query row 32sub + 16(r/8) + 8hi + r%8.
    // dP starts from -delta of its row, so that it ends as dP - delta.  S
    // starts at 0, or on partial tiles at -inf for the pairs the mask removes
    // (key kp is allowed for a row iff kp - lo <= span as unsigned numbers,
    // span = pos - lo), which makes P = 0 there: the vector part after the
    // MFMAs is the same for every tile and shares a basic block with them.
    // Padding rows (span 0, lo INT_MIN) are masked; integer arrays are read
    // as integer vectors (a bit_cast of one element of a float vector has been
    // seen to read element 0 whatever the index).
    f32x16 s, dp;
    if (full) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ro = (16 * (i >> 1) + 4 * (i & 1)) * 4;
        const u32x4 lo = *(const __attribute__((address_space(3))) u32x4*)(rowb + 2 * kQT * 4 + ro);
        const u32x4 sp = *(const __attribute__((address_space(3))) u32x4*)(rowb + 3 * kQT * 4 + ro);
#pragma unroll
        for (int e = 0; e < 4; ++e) s[4 * i + e] = ((unsigned)kp - lo[e] <= sp[e]) ? 0.f : -__builtin_inff();
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // registers 4i..4i+3: rows 16(i/2) + 4(i%2) + 0..3 of the lane's 8
      const f32x4 v = *(const __attribute__((address_space(3))) f32x4*)(rowb + kQT * 4 +
                                                                         (16 * (i >> 1) + 4 * (i & 1)) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) dp[4 * i + e] = v[e];
    }
    // Operands are read one d-slice ahead.
    bf16x8 aq[2], ao[2], bv[2];
    aq[0] = lds_read8(qn + yo[0]);
    ao[0] = lds_read8(on + yo[0]);
    bv[0] = lds_read8(vn);
#pragma unroll
    for (int kk = 0; kk < C::KREG; ++kk) {
      if (kk + 1 < C::KREG) {
        aq[(kk + 1) & 1] = lds_read8(qn + yo[kk + 1]);
        ao[(kk + 1) & 1] = lds_read8(on + yo[kk + 1]);
        bv[(kk + 1) & 1] = lds_read8(vn + (kk + 1) * 2 * kVColBytes);
      }
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[kk & 1], kreg[kk], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao[kk & 1], bv[kk & 1], dp, 0, 0, 0);
    }
    // P = exp2(c2 s - LSE log2 e), dS = P (dP - delta).
    bf16x8 pb[2], db[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // values 4i..4i+3: rows 16(i/2) + 4(i%2) + 0..3 of the lane's 8
      const int ro = (16 * (i >> 1) + 4 * (i & 1)) * 4;
      const f32x4 nl = *(const __attribute__((address_space(3))) f32x4*)(rowb + ro);
      float pr[4], ds[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int x = 4 * i + e;
        pr[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[x], p.c2, nl[e]));
        ds[e] = pr[e] * dp[x];
      }
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const bf16x2 pp = __builtin_convertvector((f32x2){pr[e], pr[e + 1]}, bf16x2);
        const bf16x2 dd = __builtin_convertvector((f32x2){ds[e], ds[e + 1]}, bf16x2);
        const int j = 4 * (i & 1) + e;
        pb[i >> 1][j] = pp[0];
        pb[i >> 1][j + 1] = pp[1];
        db[i >> 1][j] = dd[0];
        db[i >> 1][j + 1] = dd[1];
      }
    }
    // dV^T += dO^T P, dK^T += Q^T dS over the half tile's 32 query rows.
    constexpr int NG = 2 * C::DT;  // (gg, t) pairs
    // Pair m = DT*gg + t: rows +16gg, chunk group t.
    auto trd = [&](auto buf, int m) {
      const lds_char* b = to_lds(buf) + sub * 32 * C::ROW + (m / C::DT) * 16 * C::ROW;
      const int x0 = xo[m % C::DT];
      return lds_read_tr(b + x0, b + (x0 + xd));
    };
    bf16x8 to[2], tq[2];
    to[0] = trd(obuf(bc), 0);
    tq[0] = trd(qbuf(bc), 0);
#pragma unroll
    for (int m = 0; m < NG; ++m) {
      if (m + 1 < NG) {
        to[(m + 1) & 1] = trd(obuf(bc), m + 1);
        tq[(m + 1) & 1] = trd(qbuf(bc), m + 1);
      }
      const int t = m % C::DT, gg = m / C::DT;
      dva[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(to[m & 1], pb[gg], dva[t], 0, 0, 0);
      dka[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq[m & 1], db[gg], dka[t], 0, 0, 0);
    }
  };
  const int total = g * p.nqt;
  const int csh = 2 * wave;
  for (int u0 = 0; u0 < total; u0 += C::LIST) {
    const int cnt = build(u0, min(total, u0 + C::LIST));
    if (cnt == 0) continue;
    // Lane l of (lx, ly) holds list slot lb + l (0 past the end): a tile
    // takes its entries with v_readlane, not an LDS read per tile; the lane
    // vectors are refilled from LDS once per 63 tiles.
    int lb = 0, lx = 0, ly = 0;
    auto fill = [&](int b0) {
      lb = b0;
      int2 e = {0, 0};
      if (b0 + lane < cnt) e = sList[b0 + lane];
      lx = e.x;
      ly = e.y;
    };
    auto ent = [&](int j) {
      int2 e;
      e.x = __builtin_amdgcn_readlane(lx, j - lb);
      e.y = __builtin_amdgcn_readlane(ly, j - lb);
      return e;
    };
    fill(0);
    const std::integral_constant<int, 0> b0{};
    const std::integral_constant<int, 1> b1{};
    issue(b0, ent(0).x);
    wait_vmem();
    __syncthreads();
    // Tile j from buffer B while tile j+1 is copied into the other buffer.
    auto tile = [&](auto bc, int j) {
      if (j + 1 - lb >= 64) fill(j);
      if (j + 1 < cnt) issue(std::integral_constant<int, 1 - decltype(bc)::value>{}, ent(j + 1).x);
      const int cls = (int)(((unsigned)ent(j).y >> csh) & 3);
      if (cls != kSkip) {
        half(bc, 0, cls == kFull);
        half(bc, 1, cls == kFull);
      }
      wait_vmem();
      __syncthreads();
    };
    for (int j = 0; j < cnt; j += 2) {
      tile(b0, j);
      if (j + 1 < cnt) tile(b1, j + 1);
    }
  }

  // ---- accumulate into dK, dV (this lane's key; d = 32t + 8*(r/4) + 4*hi + r%4)
  // One array at a time, each read whole before it is written: dK and dV may
  // alias as far as the compiler knows, so a load of one after a store to the
  // other waits for that store's round trip; read in pairs, the update made
  // one round trip per 16-byte pair.  At d = 128 the values are first
  // regrouped through LDS so that the global accesses are whole rows.
  if constexpr (D == 128) {
    // Each 32-column slice of the wave's accumulators goes through the wave's
    // own LDS slot (the V tile's space, read by no wave after the loop's last
    // barrier), so that a global access covers 8 whole 128-byte rows instead
    // of 32 quarter rows.  Lane l then owns key 8i + l/8 of the wave and
    // columns 32t + 4(l%8) .. +3.
    constexpr int STR = 144;  // bytes per staged row (128 + 16: no bank conflicts on the writes)
    static_assert(NW * 32 * STR <= C::VTILE, "staging slots fit in the V tile's space");
    wait_vmem();              // the V copy into that space has landed (no tile may have waited for it)
    lds_char* slot = to_lds(sV) + wave * 32 * STR;
    // The lane index recomputed here, so that nothing derived from it stays
    // live across the tile loop (which uses every register).
    const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int kr = ln >> 3, c4 = 4 * (ln & 7), r32 = ln & 31, h32 = ln >> 5;
    auto acc = [&](float* base, const f32x16* a, float sc) {
      // Every address is one base pointer plus a constant, so the compiler
      // can tell the 16 accesses of an array apart and issue the loads together.
      float* rp = base + (long long)(key0 + wave * 32 + kr) * D + c4;
      f32x4 x[C::DT][4];
#pragma unroll
      for (int t = 0; t < C::DT; ++t) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const f32x4 v = {a[t][4 * rg], a[t][4 * rg + 1], a[t][4 * rg + 2], a[t][4 * rg + 3]};
          *reinterpret_cast<f32x4*>(slot + r32 * STR + (8 * rg + 4 * h32) * 4) = v;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) x[t][i] = *reinterpret_cast<const f32x4*>(slot + (8 * i + kr) * STR + c4 * 4);
      }
      f32x4 y[C::DT][4];
#pragma unroll
      for (int t = 0; t < C::DT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          y[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (wave * 32 + 8 * i + kr < nkeys) y[t][i] = *reinterpret_cast<const f32x4*>(rp + 8 * i * D + 32 * t);
        }
#pragma unroll
      for (int t = 0; t < C::DT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int e = 0; e < 4; ++e) y[t][i][e] += sc * x[t][i][e];
          if (wave * 32 + 8 * i + kr < nkeys) *reinterpret_cast<f32x4*>(rp + 8 * i * D + 32 * t) = y[t][i];
        }
    };
    acc(p.dk + ((long long)b * p.Hkv + kvh) * p.sk * D, dka, p.scale);
    acc(p.dv + ((long long)b * p.Hkv + kvh) * p.sk * D, dva, 1.f);
  } else if (kvalid) {
    auto acc = [&](float* r, const f32x16* a, float sc) {
      f32x4 x[C::DT][4];
#pragma unroll
      for (int t = 0; t < C::DT; ++t)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) x[t][rg] = *reinterpret_cast<const f32x4*>(r + 32 * t + 8 * rg + 4 * hi);
#pragma unroll
      for (int t = 0; t < C::DT; ++t)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[t][rg][e] += sc * a[t][4 * rg + e];
          *reinterpret_cast<f32x4*>(r + 32 * t + 8 * rg + 4 * hi) = x[t][rg];
        }
    };
    acc(p.dk + (((long long)b * p.Hkv + kvh) * p.sk + krow) * D, dka, p.scale);
    acc(p.dv + (((long long)b * p.Hkv + kvh) * p.sk + krow) * D, dva, 1.f);
  }
#endif
}

// ============================================================================
// dQ
// ============================================================================
// A workgroup of 8 waves owns 256 query rows (32 a wave) of one query head and
// walks the ring's 64-key tiles like the forward: per 32-key half tile,
// S^T = K Q^T and dP^T = V dO^T (the wave's rows as MFMA columns, Q and dO in
// registers), then dS^T, then dQ^T += K^T dS^T with K^T read from the K tile
// by transposing LDS reads.  K and V tiles are row-major with the swz_t chunk
// permutation (whole rows per DMA instruction, conflict-free row and
// transposed reads) and double-buffered in separate arrays with roles fixed at
// compile time, so the compiler sees that a tile's reads and the copy into
// the other buffer do not overlap.
template <int D>
struct QCfg {
  static constexpr int NW = 8;
  static constexpr int ROW = D * 2;             // bytes per K / V row
  static constexpr int CHR = D / 8;
  static constexpr int TILE = kKT * ROW;        // one K or V tile (row-major)
  static constexpr int NBLK = TILE / 1024;      // 1 KB DMA blocks per tile
  static constexpr int RPB = 1024 / ROW;        // rows per DMA block
  static constexpr int QREG = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int LIST = 2048;
  static constexpr int LOADS = (2 * NBLK) / NW;  // DMA instructions per wave per tile (wave 0: one more)
  static_assert(NW % (16 / RPB) == 0 && NBLK % (16 / RPB) == 0 && (2 * NBLK) % NW == 0, "DMA split");
};

template <int D>
__global__ __launch_bounds__(512, 1) void dq_kernel(BParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = QCfg<D>;
  constexpr int NW = C::NW;
  __shared__ __attribute__((aligned(1024))) char sK0[C::TILE];
  __shared__ __attribute__((aligned(1024))) char sK1[C::TILE];
  __shared__ __attribute__((aligned(1024))) char sV0[C::TILE];
  __shared__ __attribute__((aligned(1024))) char sV1[C::TILE];
  __shared__ __attribute__((aligned(16))) int sP0[kKT];
  __shared__ __attribute__((aligned(16))) int sP1[kKT];
  __shared__ int2 sList[C::LIST];
  __shared__ int sCnt[NW];
  __shared__ int sWb[NW][6];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int s16 = lane & 15;
  const int g = p.Hq / p.Hkv;
  const int nqt = (p.sq + NW * 32 - 1) / (NW * 32);

  int logical = xcd_logical_block();
  const int hg = logical % g;
  logical /= g;
  const int qt = p.q_order ? p.q_order[logical % nqt] : nqt - 1 - logical % nqt;
  logical /= nqt;
  const int kvh = logical % p.Hkv;
  const int b = logical / p.Hkv;
  const int h = kvh * g + hg;
  const int row = qt * NW * 32 + wave * 32 + l32;
  const bool valid = row < p.sq;
  const long long bh = (long long)b * p.Hq + h;

  // Q and dO of this lane's row as B operands (k-slots: d = 16kk + 8hi + j).
  bf16x8 qreg[C::QREG], oreg[C::QREG];
  {
    const char* qr = p.q + ((long long)b * p.q_sb + (long long)h * p.q_sh + (long long)row * p.q_ss) * 2;
    const char* orr = p.dout + ((long long)b * p.q_sb + (long long)h * p.q_sh + (long long)row * p.q_ss) * 2;
#pragma unroll
    for (int kk = 0; kk < C::QREG; ++kk) {
      qreg[kk] = __builtin_bit_cast(bf16x8, valid ? *reinterpret_cast<const u32x4*>(qr + (16 * kk + 8 * hi) * 2)
                                                  : u32x4{0, 0, 0, 0});
      oreg[kk] = __builtin_bit_cast(bf16x8, valid ? *reinterpret_cast<const u32x4*>(orr + (16 * kk + 8 * hi) * 2)
                                                  : u32x4{0, 0, 0, 0});
    }
  }
  const int qp = valid ? p.q_pos[row] : -1;
  const int ql = valid ? (p.q_lo ? p.q_lo[row] : 0) : INT_MAX;
  const float nl2 = valid ? p.nl2[bh * p.sq_pad + row] : 0.f;
  const float ndl = valid ? p.dlt[bh * p.sq_pad + row] : 0.f;
  wave_row_bounds(wave, lane, valid, qp, ql, sWb);
  __syncthreads();

  const long long k_row_bytes = p.k_ss * 2;
  const long long v_row_bytes = p.v_ss * 2;
  // DMA: blocks wave, wave + NW, ... of the K and V tiles; lane l fills slot
  // l % CHR of row l / CHR of its block (all of a wave's blocks share one
  // swizzle pattern).
  const int lrow = lane / C::CHR;
  const int lslot = 16 * swz_t<C::CHR>(C::RPB * (wave % C::NBLK) + lrow, lane % C::CHR);
  const int voffK = (int)(lrow * k_row_bytes) + lslot;
  const int voffV = (int)(lrow * v_row_bytes) + lslot;
  // Row reads (A of S^T = K Q^T and dP^T = V dO^T): key key_perm(l32) (+32
  // sub), logical chunk 2kk + hi, at byte nrow*ROW + ((32 kk) ^ nY).
  const int nrow = key_perm(l32);
  const int nY = 16 * (hi ^ swz_t<C::CHR>(nrow, 0));
  // Transposed reads of K (A of dQ^T += K^T dS^T): lane s16 of its 16-lane
  // group reads key 8hi + 4h + s16/4 (+16gg + 32sub) at column 32t +
  // 16*(bit 4 of lane) + 4*(s16%4): byte tP[h] + ((64 t) ^ tA), kept as
  // xo[t] = tP[0] + ((64 t) ^ tA) and the distance xd = tP[1] - tP[0].
  int tP[2], tA;
  {
    const int cl = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int r = 8 * hi + 4 * hh + (s16 >> 2);
      const int f = swz_t<C::CHR>(r, 0);
      tP[hh] = r * C::ROW + 16 * (cl ^ (f & 3)) + 8 * (s16 & 1);
      tA = 64 * (f >> 2);
    }
  }

  // Row reads are a per-lane offset yoff(kk) plus a constant (buffer address
  // and half-tile offset) that the DS offset field holds: the four K/V tiles
  // lie in the first 64 KiB of LDS.  With ROW = 256 the offsets of slices
  // 4..7 are those of slices 0..3 with bit 7 flipped.  The offsets pass
  // through an empty asm in place at each half tile so that the compiler does
  // not hoist offset + constant out of the loop as one register per read.
  constexpr int NYO = C::QREG > 4 ? 4 : C::QREG;
  static_assert(C::QREG <= 4 || C::ROW == 256, "offset reuse");
  int yo[NYO];
#pragma unroll
  for (int kk = 0; kk < NYO; ++kk) yo[kk] = nrow * C::ROW + ((32 * kk) ^ nY);
  auto yoff = [&](int kk) { return kk < NYO ? yo[kk] : (yo[kk - NYO] ^ 128); };
  int xo[C::DT];
#pragma unroll
  for (int t = 0; t < C::DT; ++t) xo[t] = tP[0] + ((64 * t) ^ tA);
  int xd = tP[1] - tP[0];
  auto refresh = [&]() {
#pragma unroll
    for (int kk = 0; kk < NYO; ++kk) asm volatile("" : "+v"(yo[kk]));
#pragma unroll
    for (int t = 0; t < C::DT; ++t) asm volatile("" : "+v"(xo[t]));
    asm volatile("" : "+v"(xd));
  };

  const char* kbase = p.k + ((long long)b * p.k_sb + (long long)kvh * p.k_sh) * 2;
  const char* vbase = p.v + ((long long)b * p.v_sb + (long long)kvh * p.v_sh) * 2;
  const __amdgpu_buffer_rsrc_t rsP = __builtin_amdgcn_make_buffer_rsrc((void*)p.kpos_pad, 0, 0x7fffffff, kBufferFlags);

  auto kbuf = [&](auto bc) -> char* { if constexpr (decltype(bc)::value) return sK1; else return sK0; };
  auto vbuf = [&](auto bc) -> char* { if constexpr (decltype(bc)::value) return sV1; else return sV0; };
  auto pbuf = [&](auto bc) -> int* { if constexpr (decltype(bc)::value) return sP1; else return sP0; };

  // Copies key tile e (src | i << 8) into buffer B: LOADS blocks per wave, and
  // the padded key positions (wave 0).
  auto issue = [&](auto bc, int e) {
    const int src = e & 0xFF, i = (e >> 8) & 0xFFFF;
    const int tile = src * p.tpr + i;
    const int r0 = src * p.R + i * kKT;
    const int nval = min(kKT, p.R - i * kKT);
    const __amdgpu_buffer_rsrc_t rsK = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kbase + (long long)r0 * k_row_bytes), 0, (int)(nval * k_row_bytes), kBufferFlags);
    const __amdgpu_buffer_rsrc_t rsV = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vbase + (long long)r0 * v_row_bytes), 0, (int)(nval * v_row_bytes), kBufferFlags);
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) {
      const int bi = wave + NW * j;
      const int ib = bi % C::NBLK;
      if (bi < C::NBLK)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsK, (lds_ptr_t)(kbuf(bc) + ib * 1024), 16, voffK,
                                                 (int)(C::RPB * ib * k_row_bytes), 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsV, (lds_ptr_t)(vbuf(bc) + ib * 1024), 16, voffV,
                                                 (int)(C::RPB * ib * v_row_bytes), 0, 0);
    }
    if (wave == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsP, (lds_ptr_t)pbuf(bc), 4, lane * 4, tile * kKT * 4, 0, 0);
  };

  f32x16 dqa[C::DT];
#pragma unroll
  for (int t = 0; t < C::DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[t][r] = 0.f;

  // One half tile (sub: keys 32sub..32sub+31) of the tile in buffer buf.
  auto half = [&](auto bc, int sub, bool full) {
    refresh();
    const lds_char* kn = to_lds(kbuf(bc)) + sub * 32 * C::ROW;
    const lds_char* vn = to_lds(vbuf(bc)) + sub * 32 * C::ROW;
    // S^T, dP^T: register r is key 32sub + 16(r/8) + 8hi + r%8.  S^T starts
    // at 0, or on partial tiles at -inf for the keys outside [q_lo, q_pos] of
    // the lane's row, which makes P = 0 there: the vector part after the MFMAs
    // is the same for every tile and shares a basic block with them.
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) dp[r] = 0.f;
    if (full) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
    } else {
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int* kpp = pbuf(bc) + 32 * sub + 16 * gg + 8 * hi;
        const int4 k0 = *reinterpret_cast<const int4*>(kpp);
        const int4 k1 = *reinterpret_cast<const int4*>(kpp + 4);
        const int kv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) s[8 * gg + j] = (kv[j] >= ql && kv[j] <= qp) ? 0.f : -__builtin_inff();
      }
    }
#pragma unroll
    for (int kk = 0; kk < C::QREG; ++kk) {
      const int y = yoff(kk);
      const bf16x8 ak = lds_read8(kn + y);
      const bf16x8 av = lds_read8(vn + y);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qreg[kk], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, oreg[kk], dp, 0, 0, 0);
    }
    // dS^T = P^T (dP^T - delta), P^T = exp2(c2 s - LSE log2 e).
    bf16x8 db[2];
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        float ds[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 8 * gg + j + e;
          ds[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], p.c2, nl2)) * (dp[r] + ndl);
        }
        const bf16x2 dd = __builtin_convertvector((f32x2){ds[0], ds[1]}, bf16x2);
        db[gg][j] = dd[0];
        db[gg][j + 1] = dd[1];
      }
    }
    // dQ^T += K^T dS^T over the half tile's 32 keys.
    const lds_char* kt = to_lds(kbuf(bc)) + sub * 32 * C::ROW;
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int t = 0; t < C::DT; ++t) {
        const lds_char* kg = kt + gg * 16 * C::ROW;
        const bf16x8 a = lds_read_tr(kg + xo[t], kg + (xo[t] + xd));
        dqa[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, db[gg], dqa[t], 0, 0, 0);
      }
  };

  const int total = p.cp * p.tpr;
  const int csh = 2 * wave;
  for (int u0 = 0; u0 < total; u0 += C::LIST) {
    const int cnt = build_key_list<kKT, NW, C::LIST>(p.kbounds, p.tpr, p.R, p.rank, p.cp, u0, min(total, u0 + C::LIST), tid,
                                            wave, lane, sWb, sList, sCnt);
    if (cnt == 0) continue;
    // Lane l of (lx, ly) holds list slot lb + l (0 past the end): a tile
    // takes its entries with v_readlane, not an LDS read per tile; the lane
    // vectors are refilled from LDS once per 63 tiles.
    int lb = 0, lx = 0, ly = 0;
    auto fill = [&](int b0) {
      lb = b0;
      int2 e = {0, 0};
      if (b0 + lane < cnt) e = sList[b0 + lane];
      lx = e.x;
      ly = e.y;
    };
    auto ent = [&](int j) {
      int2 e;
      e.x = __builtin_amdgcn_readlane(lx, j - lb);
      e.y = __builtin_amdgcn_readlane(ly, j - lb);
      return e;
    };
    fill(0);
    const std::integral_constant<int, 0> b0{};
    const std::integral_constant<int, 1> b1{};
    issue(b0, ent(0).x);
    wait_vmem();
    __syncthreads();
    // Tile j from buffer B while tile j+1 is copied into the other buffer.
    auto tile = [&](auto bc, int j) {
      if (j + 1 - lb >= 64) fill(j);
      if (j + 1 < cnt) issue(std::integral_constant<int, 1 - decltype(bc)::value>{}, ent(j + 1).x);
      const int cls = (int)(((unsigned)ent(j).y >> csh) & 3);
      if (cls != kSkip) {
        half(bc, 0, cls == kFull);
        half(bc, 1, cls == kFull);
      }
      wait_vmem();
      __syncthreads();
    };
    for (int j = 0; j < cnt; j += 2) {
      tile(b0, j);
      if (j + 1 < cnt) tile(b1, j + 1);
    }
  }

  // Accumulate into dQ.  At d = 128 the values are first regrouped through
  // LDS (the K/V tiles' space, read by no wave after the loop's last barrier;
  // three 4.5 KB slots per 16 KB tile), one 32-column slice at a time, so
  // that lane l owns row 8i + l/8 of the wave and columns 32t + 4(l%8) .. +3,
  // and each global access covers 8 whole 128-byte rows.
  if constexpr (D == 128) {
    constexpr int STR = 144;  // bytes per staged row (128 + 16: no bank conflicts on the writes)
    static_assert(3 * 32 * STR <= C::TILE && NW <= 9, "three staging slots per tile buffer");
    wait_vmem();
    char* sb = wave < 3 ? sK0 : (wave < 6 ? sK1 : sV0);
    lds_char* slot = to_lds(sb) + (wave % 3) * 32 * STR;
    // The lane index recomputed here, so that nothing derived from it stays
    // live across the tile loop.
    const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int kr = ln >> 3, c4 = 4 * (ln & 7), r32 = ln & 31, h32 = ln >> 5;
    const int row0 = qt * NW * 32 + wave * 32;  // the wave's first row
    float* rp = p.dq + (bh * p.sq + row0 + kr) * D + c4;
    f32x4 x[C::DT][4];
#pragma unroll
    for (int t = 0; t < C::DT; ++t) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const f32x4 v = {dqa[t][4 * rg], dqa[t][4 * rg + 1], dqa[t][4 * rg + 2], dqa[t][4 * rg + 3]};
        *reinterpret_cast<f32x4*>(slot + r32 * STR + (8 * rg + 4 * h32) * 4) = v;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) x[t][i] = *reinterpret_cast<const f32x4*>(slot + (8 * i + kr) * STR + c4 * 4);
    }
    f32x4 y[C::DT][4];
#pragma unroll
    for (int t = 0; t < C::DT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (row0 + 8 * i + kr < p.sq) y[t][i] = *reinterpret_cast<const f32x4*>(rp + 8 * i * D + 32 * t);
      }
#pragma unroll
    for (int t = 0; t < C::DT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[t][i][e] += p.scale * x[t][i][e];
        if (row0 + 8 * i + kr < p.sq) *reinterpret_cast<f32x4*>(rp + 8 * i * D + 32 * t) = y[t][i];
      }
  } else if (valid) {
    float* dqr = p.dq + (bh * p.sq + row) * D;
#pragma unroll
    for (int t = 0; t < C::DT; ++t)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int dd = 32 * t + 8 * rg + 4 * hi;
        f32x4 q4 = *reinterpret_cast<f32x4*>(dqr + dd);
#pragma unroll
        for (int e = 0; e < 4; ++e) q4[e] += p.scale * dqa[t][4 * rg + e];
        *reinterpret_cast<f32x4*>(dqr + dd) = q4;
      }
  }
#endif
}

template <int D>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  const BwdWorkspace w = bwd_workspace_layout(a.b, a.hq, a.hkv, a.d, a.sq, a.sk, a.cp);
  char* ws = static_cast<char*>(a.ws);
  BParams p{};
  p.q = static_cast<const char*>(a.q);
  p.k = static_cast<const char*>(a.k);
  p.v = static_cast<const char*>(a.v);
  p.dout = static_cast<const char*>(a.dout);
  p.q_pos = a.q_pos;
  p.q_lo = a.q_lo;
  p.k_pos = a.k_pos;
  p.kbounds = reinterpret_cast<const int4*>(ws + w.kbounds_off);
  p.kpos_pad = reinterpret_cast<const int*>(ws + w.kpos_off);
  p.qbounds = reinterpret_cast<const int4*>(ws + w.qbounds_off);
  p.qholes = reinterpret_cast<const int2*>(ws + w.qholes_off);
  p.qlo_pad = reinterpret_cast<const int*>(ws + w.qlo_off);
  p.qspan_pad = reinterpret_cast<const int*>(ws + w.qspan_off);
  p.nl2 = reinterpret_cast<const float*>(ws + w.nl2_off);
  p.dlt = reinterpret_cast<const float*>(ws + w.dlt_off);
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.q_sb = a.q_str[0];
  p.q_sh = a.q_str[1];
  p.q_ss = a.q_str[2];
  p.k_sb = a.k_str[0];
  p.k_sh = a.k_str[1];
  p.k_ss = a.k_str[2];
  p.v_sb = a.v_str[0];
  p.v_sh = a.v_str[1];
  p.v_ss = a.v_str[2];
  p.sq_pad = (int)w.sq_pad;
  p.B = a.b;
  p.Hq = a.hq;
  p.Hkv = a.hkv;
  p.sq = a.sq;
  p.sk = a.sk;
  p.cp = a.cp;
  p.rank = a.rank;
  p.R = a.rows_per_rank;
  p.tpr = (a.rows_per_rank + kKT - 1) / kKT;
  p.nqt = (int)(w.sq_pad / kQT);
  p.c2 = a.scale * kLog2e;
  p.scale = a.scale;
  const int ntiles = a.cp * p.tpr;
  if (ntiles > 0) {
    hipLaunchKernelGGL(key_prep_kernel, dim3(ntiles), dim3(64), 0, stream, p,
                       reinterpret_cast<int4*>(ws + w.kbounds_off), reinterpret_cast<int*>(ws + w.kpos_off));
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(query_prep_kernel, dim3(p.nqt, a.b * a.hq), dim3(64), 0, stream, p, a.lse, a.delta,
                     reinterpret_cast<int4*>(ws + w.qbounds_off), reinterpret_cast<int2*>(ws + w.qholes_off),
                     reinterpret_cast<int*>(ws + w.qlo_off),
                     reinterpret_cast<int*>(ws + w.qspan_off), reinterpret_cast<float*>(ws + w.nl2_off),
                     reinterpret_cast<float*>(ws + w.dlt_off));
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (ntiles == 0) return hipSuccess;
  const int tg = (a.rows_per_rank + kKeysPerWg - 1) / kKeysPerWg;
  // Dispatch orders, most work first: the work per key group (and, under
  // document masks, per query tile) is uneven and does not follow the index,
  // so in index order the longest workgroups could start last.  Dense rings
  // of many key groups are left in index order, which already puts the
  // heaviest groups (the shards' early chunks) first: sorted, 131072 tokens
  // ran 0.1-0.9% slower; 32768 tokens (128 groups) ran 2% faster.
  if (bwd_kv_order(a.sk, a.cp) && (a.q_lo != nullptr || a.cp * tg <= kKvOrderDenseGroups)) {
    int* cost = reinterpret_cast<int*>(ws + w.kvcost_off);
    const int ng = a.cp * tg;
    hipLaunchKernelGGL(kv_cost_kernel, dim3(ng), dim3(512), 0, stream, p, cost);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    if (hipError_t e = launch_order_sort(cost, ng, cost + ng, stream); e != hipSuccess) return e;
    p.kv_order = cost + ng;
  }
  if (a.q_lo != nullptr && bwd_q_order(a.sq)) {
    int* cost = reinterpret_cast<int*>(ws + w.qcost_off);
    const int n = (a.sq + 255) / 256;
    if (hipError_t e = launch_dq_order(a.q_pos, a.q_lo, p.kbounds, a.sq, a.rows_per_rank, p.tpr, a.rank, a.cp, cost,
                                       cost + n, stream);
        e != hipSuccess)
      return e;
    p.q_order = cost + n;
  }
  const long long nkv = (long long)a.cp * tg * a.hkv * a.b;
  hipLaunchKernelGGL((dkdv_kernel<D>), dim3((unsigned)nkv), dim3(512), 0, stream, p);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int nqt256 = (a.sq + 255) / 256;
  const long long nq = (long long)nqt256 * a.hq * a.b;
  hipLaunchKernelGGL((dq_kernel<D>), dim3((unsigned)nq), dim3(512), 0, stream, p);
  return hipGetLastError();
}

}  // namespace bwdk

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  return a.d == 64 ? bwdk::launch_bwd_t<64>(a, stream) : bwdk::launch_bwd_t<128>(a, stream);
}

namespace {
template <int D, typename OT>
hipError_t launch_delta_t(const BwdArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.b * a.hq * a.sq;
  const long long nblk = (rows + bwdk::kDeltaRowsPerBlock - 1) / bwdk::kDeltaRowsPerBlock;
  hipLaunchKernelGGL((bwdk::delta_kernel<D, OT>), dim3((unsigned)nblk), dim3(256), 0, stream,
                     static_cast<const char*>(a.dout), (long long)a.q_str[0], (long long)a.q_str[1],
                     (long long)a.q_str[2], static_cast<const OT*>(a.o), (long long)a.o_str[0], (long long)a.o_str[1],
                     (long long)a.o_str[2], a.delta_out, a.hq, a.sq, rows);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_delta(const BwdArgs& a, hipStream_t stream) {
  if (a.out_dtype == CP_BF16)
    return a.d == 64 ? launch_delta_t<64, __bf16>(a, stream) : launch_delta_t<128, __bf16>(a, stream);
  return a.d == 64 ? launch_delta_t<64, float>(a, stream) : launch_delta_t<128, float>(a, stream);
}

}  // namespace cpattn
