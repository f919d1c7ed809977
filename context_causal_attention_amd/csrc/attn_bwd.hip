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
//     dK^T += Q^T dS (query rows read in the permuted order of key_perm).
//   * dq_kernel: a workgroup owns 256 query rows (32 a wave) of one head and
//     walks the ring's key tiles like the forward; S^T = K Q^T, dP^T = V dO^T,
//     dQ^T += K^T dS^T, with Q and dO of the wave's rows resident.
// Operand tiles are copied HBM -> LDS by buffer loads with the LDS-direct bit;
// transposed copies (Q^T, dO^T, K^T) come from a preparation pass.
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
  const int4* kbounds;   // per 64-key tile {min pos, max pos, valid rows, 0}
  const int* kpos_pad;   // per key slot, padding = kInvalidKey
  const char* kt;        // bf16 K^T [b][hkv][d][kt_row]
  const int4* qbounds;   // per 64-row query tile {min pos, max pos, min lo, max lo}
  const int* qpos_pad;   // per query slot [sq_pad], padding = -1
  const int* qlo_pad;    // padding = INT_MAX
  const float* lse2;     // [b][hq][sq_pad]: LSE * log2(e), 0 in padding
  const float* dlt;      // [b][hq][sq_pad]: delta, 0 in padding
  const char* qt;        // bf16 Q^T  [b][hq][d][sq_pad]
  const char* dot;       // bf16 dO^T [b][hq][d][sq_pad]
  float* dq;             // fp32 [b, hq, sq, d] contiguous, accumulated
  float* dk;             // fp32 [b, hkv, sk, d] contiguous, accumulated
  float* dv;
  long long q_sb, q_sh, q_ss, k_sb, k_sh, k_ss, v_sb, v_sh, v_ss;
  long long kt_row;      // elements per K^T row
  int sq_pad;            // query rows per (b, head), padded to kQT
  int B, Hq, Hkv, sq, sk, cp, rank, R, tpr, nqt;
  float c2;              // scale * log2(e)
  float scale;
};

// ============================================================================
// Preparation
// ============================================================================
// Key side, per 64-key tile of a rank's shard: position bounds, padded key
// positions and K^T.
template <int D>
__global__ __launch_bounds__(256) void key_prep_kernel(BParams p, int4* __restrict__ kbounds, int* __restrict__ kpos_pad,
                                                       __bf16* __restrict__ kt) {
  const int tile = blockIdx.x;
  const int src = tile / p.tpr;
  const int i = tile - src * p.tpr;
  const int r0 = src * p.R + i * kKT;
  const int nval = min(kKT, p.R - i * kKT);
  const int tid = threadIdx.x;
  if (blockIdx.y == 0 && tid < 64) {
    const bool ok = tid < nval;
    const int kp = ok ? p.k_pos[r0 + tid] : 0;
    const int mn = wave_min(ok ? kp : INT_MAX);
    const int mx = wave_max(ok ? kp : INT_MIN);
    if (tid == 0) kbounds[tile] = int4{mn, mx, nval, 0};
    kpos_pad[tile * kKT + tid] = ok ? kp : kInvalidKey;
  }
  __shared__ __bf16 s[kKT][D + 8];
  const int b = blockIdx.y / p.Hkv, kvh = blockIdx.y % p.Hkv;
  const char* kb = p.k + ((long long)b * p.k_sb + (long long)kvh * p.k_sh) * 2;
  constexpr int CH = D / 8;
  for (int c = tid; c < kKT * CH; c += 256) {
    const int r = c / CH, ch = c % CH;
    const u32x4 raw = r < nval ? *reinterpret_cast<const u32x4*>(kb + ((long long)(r0 + r) * p.k_ss + ch * 8) * 2)
                               : u32x4{0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(&s[r][ch * 8]) = raw;
  }
  __syncthreads();
  __bf16* out = kt + ((long long)blockIdx.y * D) * p.kt_row + (long long)tile * kKT;
  for (int c = tid; c < D * (kKT / 8); c += 256) {
    const int dd = c / (kKT / 8), kc = c % (kKT / 8);
    bf16x8 w;
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = s[kc * 8 + j][dd];
    *reinterpret_cast<bf16x8*>(out + (long long)dd * p.kt_row + kc * 8) = w;
  }
}

// Query side, per 64-row tile of one (batch, query head): Q^T and dO^T, LSE in
// base 2 and delta padded to the tile grid; for the first (batch, head) also the
// tile's position bounds and the padded positions.
template <int D>
__global__ __launch_bounds__(256) void query_prep_kernel(BParams p, const float* __restrict__ lse,
                                                         const float* __restrict__ delta, int4* __restrict__ qbounds,
                                                         int* __restrict__ qpos_pad, int* __restrict__ qlo_pad,
                                                         float* __restrict__ lse2, float* __restrict__ dlt,
                                                         __bf16* __restrict__ qt, __bf16* __restrict__ dot) {
  const int tile = blockIdx.x;
  const int r0 = tile * kQT;
  const int nval = min(kQT, p.sq - r0);
  const int tid = threadIdx.x;
  const int bh = blockIdx.y;  // b * Hq + h
  if (bh == 0 && tid < 64) {
    const bool ok = tid < nval;
    const int qp = ok ? p.q_pos[r0 + tid] : -1;
    const int ql = ok ? (p.q_lo ? p.q_lo[r0 + tid] : 0) : INT_MAX;
    const int a = wave_min(ok ? qp : INT_MAX), b = wave_max(ok ? qp : INT_MIN);
    const int c = wave_min(ok ? ql : INT_MAX), d = wave_max(ok ? ql : INT_MIN);
    if (tid == 0) qbounds[tile] = int4{a, b, c, d};
    qpos_pad[r0 + tid] = qp;
    qlo_pad[r0 + tid] = ql;
  }
  if (tid < 64) {
    const bool ok = tid < nval;
    const long long idx = (long long)bh * p.sq + r0 + tid;
    lse2[(long long)bh * p.sq_pad + r0 + tid] = ok ? lse[idx] * kLog2e : 0.f;
    dlt[(long long)bh * p.sq_pad + r0 + tid] = ok ? delta[idx] : 0.f;
  }
  __shared__ __bf16 s[2][kQT][D + 8];
  const int b = bh / p.Hq, h = bh % p.Hq;
  constexpr int CH = D / 8;
  for (int c = tid; c < 2 * kQT * CH; c += 256) {
    const int which = c / (kQT * CH);
    const int cc = c % (kQT * CH);
    const int r = cc / CH, ch = cc % CH;
    const char* src = which ? p.dout : p.q;
    const u32x4 raw = r < nval ? *reinterpret_cast<const u32x4*>(
                                     src + ((long long)b * p.q_sb + (long long)h * p.q_sh + (long long)(r0 + r) * p.q_ss + ch * 8) * 2)
                               : u32x4{0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(&s[which][r][ch * 8]) = raw;
  }
  __syncthreads();
  for (int c = tid; c < 2 * D * (kQT / 8); c += 256) {
    const int which = c / (D * (kQT / 8));
    const int cc = c % (D * (kQT / 8));
    const int dd = cc / (kQT / 8), qc = cc % (kQT / 8);
    bf16x8 w;
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = s[which][qc * 8 + j][dd];
    __bf16* out = (which ? dot : qt) + ((long long)bh * D + dd) * p.sq_pad + r0 + qc * 8;
    *reinterpret_cast<bf16x8*>(out) = w;
  }
}

// delta_q = sum_d dO[q, d] * O[q, d]; one half-wave (32 lanes) per row.
template <int D, typename OT>
__global__ __launch_bounds__(256) void delta_kernel(const char* __restrict__ dout, long long do_sb, long long do_sh,
                                                    long long do_ss, const OT* __restrict__ o, long long o_sb,
                                                    long long o_sh, long long o_ss, float* __restrict__ delta, int Hq,
                                                    int sq, long long rows) {
  const long long r = ((long long)blockIdx.x * 256 + threadIdx.x) / 32;
  const int lane = threadIdx.x & 31;
  float acc = 0.f;
  if (r < rows) {
    const long long bh = r / sq;
    const int i = (int)(r - bh * sq);
    const int b = (int)(bh / Hq), h = (int)(bh % Hq);
    constexpr int PER = D / 32;  // elements per lane
    const __bf16* dp = reinterpret_cast<const __bf16*>(dout) + (long long)b * do_sb + (long long)h * do_sh +
                       (long long)i * do_ss + lane * PER;
    const OT* op = o + (long long)b * o_sb + (long long)h * o_sh + (long long)i * o_ss + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc += (float)dp[e] * (float)op[e];
  }
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 32);
  if (r < rows && lane == 0) delta[r] = acc;
}

// ============================================================================
// dK, dV
// ============================================================================
template <int D>
struct KvCfg {
  static constexpr int NW = 4;
  static constexpr int ROW = D * 2;            // bytes per row of the Q / dO tiles
  static constexpr int CHR = D / 8;            // 16-byte chunks per such row
  static constexpr int TROW = kQT * 2;         // bytes per row of the Q^T / dO^T tiles (128)
  static constexpr int TCHR = kQT / 8;         // 8
  static constexpr int RBYTES = kQT * ROW;     // a row-major tile
  static constexpr int TBYTES = D * TROW;      // a transposed tile
  static constexpr int RPW = RBYTES / 1024 / NW;
  static constexpr int TPW = TBYTES / 1024 / NW;
  static constexpr int KREG = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int LIST = 1024;
};

template <int D>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(BParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = KvCfg<D>;
  constexpr int NW = C::NW;
  __shared__ __attribute__((aligned(1024))) char sQ[2][C::RBYTES];
  __shared__ __attribute__((aligned(1024))) char sDO[2][C::RBYTES];
  __shared__ __attribute__((aligned(1024))) char sQT[2][C::TBYTES];
  __shared__ __attribute__((aligned(1024))) char sDOT[2][C::TBYTES];
  __shared__ __attribute__((aligned(16))) float sL[2][kQT];
  __shared__ __attribute__((aligned(16))) float sDl[2][kQT];
  __shared__ __attribute__((aligned(16))) int sQp[2][kQT];
  __shared__ __attribute__((aligned(16))) int sQl[2][kQT];
  __shared__ int2 sList[C::LIST];
  __shared__ int sCnt[NW];
  __shared__ int sKb[NW][3];  // per wave: min key pos, max key pos, all keys valid

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int g = p.Hq / p.Hkv;

  // ---- work item: 128 keys of rank src's shard, for one (batch, kv head) ----
  const int t128 = (p.R + 127) / 128;  // 128-key groups per shard
  int logical = xcd_logical_block();
  const int grp = logical % (p.cp * t128);
  logical /= p.cp * t128;
  const int kvh = logical % p.Hkv;
  const int b = logical / p.Hkv;
  const int src = grp / t128;
  const int ig = grp - src * t128;
  const int kloc = ig * 128 + wave * 32 + l32;   // row within the shard
  const bool kvalid = kloc < p.R;
  const int krow = src * p.R + kloc;             // row in k_all
  const int kp = kvalid ? p.k_pos[krow] : kInvalidKey;

  // K and V of this lane's key as B operands (k-slots: d = 16kk + 8hi + j).
  bf16x8 kreg[C::KREG], vreg[C::KREG];
  {
    const char* kr = p.k + ((long long)b * p.k_sb + (long long)kvh * p.k_sh + (long long)krow * p.k_ss) * 2;
    const char* vr = p.v + ((long long)b * p.v_sb + (long long)kvh * p.v_sh + (long long)krow * p.v_ss) * 2;
#pragma unroll
    for (int kk = 0; kk < C::KREG; ++kk) {
      kreg[kk] = __builtin_bit_cast(bf16x8, kvalid ? *reinterpret_cast<const u32x4*>(kr + (16 * kk + 8 * hi) * 2)
                                                   : u32x4{0, 0, 0, 0});
      vreg[kk] = __builtin_bit_cast(bf16x8, kvalid ? *reinterpret_cast<const u32x4*>(vr + (16 * kk + 8 * hi) * 2)
                                                   : u32x4{0, 0, 0, 0});
    }
  }
  {
    const int a = wave_min(kvalid ? kp : INT_MAX);
    const int c = wave_max(kvalid ? kp : INT_MIN);
    const bool all_valid = __all(kvalid);
    if (lane == 0) {
      sKb[wave][0] = a;
      sKb[wave][1] = c;
      sKb[wave][2] = all_valid ? 1 : 0;
    }
  }
  __syncthreads();

  // ---- per-lane constant addresses ----------------------------------------
  int voffR[C::RPW], voffT[C::TPW];
  const long long q_row_bytes = p.q_ss * 2;
  const long long t_row_bytes = (long long)p.sq_pad * 2;
#pragma unroll
  for (int j = 0; j < C::RPW; ++j) {
    const int c = (wave + NW * j) * 64 + lane;
    const int r = c / C::CHR, ph = c % C::CHR;
    voffR[j] = (int)(r * q_row_bytes) + 16 * swz<C::CHR>(r, ph);
  }
#pragma unroll
  for (int j = 0; j < C::TPW; ++j) {
    const int c = (wave + NW * j) * 64 + lane;
    const int r = c / C::TCHR, ph = c % C::TCHR;
    voffT[j] = (int)(r * t_row_bytes) + 16 * swz<C::TCHR>(r, ph);
  }
  const int qrow = key_perm(l32);  // A-operand row of the row-major tiles
  int raddr[C::KREG];
#pragma unroll
  for (int kk = 0; kk < C::KREG; ++kk) raddr[kk] = qrow * C::ROW + 16 * swz<C::CHR>(qrow, 2 * kk + hi);
  int taddr[4];
#pragma unroll
  for (int kg = 0; kg < 4; ++kg) taddr[kg] = l32 * C::TROW + 16 * swz<C::TCHR>(l32, 2 * kg + hi);

  // ---- list of (query head, query tile) pairs this workgroup needs ---------
  // Slot u = hg * nqt + t.  Class per wave from the tile bounds and the wave's
  // key bounds: skip when no key of the wave lies in [min lo, max pos], full
  // when every key lies in [max lo, min pos] for every row.
  auto build = [&](int u0, int u1) {
    int cnt = 0;
    for (int base = u0; base < u1; base += NW * 64) {
      const int u = base + tid;
      bool act = false;
      int2 entry = {0, 0};
      if (u < u1) {
        const int t = u % p.nqt;
        const int4 qb = p.qbounds[t];
        const bool tile_full = (t + 1) * kQT <= p.sq;
        entry.x = u;
        unsigned bits = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const int kmn = sKb[w][0], kmx = sKb[w][1];
          int cls = kSkip;
          if (kmn != INT_MAX && kmn <= qb.y && kmx >= qb.z)
            cls = (sKb[w][2] && tile_full && kmx <= qb.x && kmn >= qb.w) ? kFull : kPartial;
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

  const __amdgpu_buffer_rsrc_t rsL = __builtin_amdgcn_make_buffer_rsrc((void*)p.lse2, 0, 0x7fffffff, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsD = __builtin_amdgcn_make_buffer_rsrc((void*)p.dlt, 0, 0x7fffffff, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsQp = __builtin_amdgcn_make_buffer_rsrc((void*)p.qpos_pad, 0, 0x7fffffff, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsQl = __builtin_amdgcn_make_buffer_rsrc((void*)p.qlo_pad, 0, 0x7fffffff, kBufferFlags);

  // Copies query tile (head h, tile t) into buffer `buf`.
  auto issue = [&](int buf, int e) __attribute__((always_inline)) {
    const int hg = e / p.nqt, t = e - (e / p.nqt) * p.nqt;
    const int h = kvh * g + hg;
    const int r0 = t * kQT;
    const int nval = min(kQT, p.sq - r0);
    const long long bh = (long long)b * p.Hq + h;
    const __amdgpu_buffer_rsrc_t rsQ = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.q + ((long long)b * p.q_sb + (long long)h * p.q_sh + (long long)r0 * p.q_ss) * 2), 0,
        (int)(nval * q_row_bytes), kBufferFlags);
    const __amdgpu_buffer_rsrc_t rsO = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.dout + ((long long)b * p.q_sb + (long long)h * p.q_sh + (long long)r0 * p.q_ss) * 2), 0,
        (int)(nval * q_row_bytes), kBufferFlags);
    const __amdgpu_buffer_rsrc_t rsQT = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.qt + (bh * D * p.sq_pad + r0) * 2), 0, (int)(D * t_row_bytes), kBufferFlags);
    const __amdgpu_buffer_rsrc_t rsOT = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.dot + (bh * D * p.sq_pad + r0) * 2), 0, (int)(D * t_row_bytes), kBufferFlags);
#pragma unroll
    for (int j = 0; j < C::RPW; ++j) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsQ, (lds_ptr_t)(&sQ[buf][0] + (wave + NW * j) * 1024), 16, voffR[j], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsO, (lds_ptr_t)(&sDO[buf][0] + (wave + NW * j) * 1024), 16, voffR[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < C::TPW; ++j) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsQT, (lds_ptr_t)(&sQT[buf][0] + (wave + NW * j) * 1024), 16, voffT[j], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsOT, (lds_ptr_t)(&sDOT[buf][0] + (wave + NW * j) * 1024), 16, voffT[j], 0, 0, 0);
    }
    if (wave == 0) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsL, (lds_ptr_t)&sL[buf][0], 4, lane * 4, (int)((bh * p.sq_pad + r0) * 4), 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsD, (lds_ptr_t)&sDl[buf][0], 4, lane * 4, (int)((bh * p.sq_pad + r0) * 4), 0, 0);
    } else if (wave == 1) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsQp, (lds_ptr_t)&sQp[buf][0], 4, lane * 4, r0 * 4, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsQl, (lds_ptr_t)&sQl[buf][0], 4, lane * 4, r0 * 4, 0, 0);
    }
  };

  auto compute = [&](int buf, int cls) __attribute__((always_inline)) {
    if (cls == kSkip) return;
    const char* q_t = &sQ[buf][0];
    const char* do_t = &sDO[buf][0];
    const char* qt_t = &sQT[buf][0];
    const char* dot_t = &sDOT[buf][0];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      // S = Q K^T and dP = dO V^T for 32 query rows (register r: row 32*sub + 16*(r/8) + 8*hi + r%8)
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int kk = 0; kk < C::KREG; ++kk) {
        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(q_t + raddr[kk] + sub * 32 * C::ROW);
        const bf16x8 ao = *reinterpret_cast<const bf16x8*>(do_t + raddr[kk] + sub * 32 * C::ROW);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kreg[kk], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, vreg[kk], dp, 0, 0, 0);
      }
      bf16x8 pb[2], db[2];
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int q0 = 32 * sub + 16 * gg + 8 * hi;
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(&sL[buf][q0]);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(&sL[buf][q0 + 4]);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(&sDl[buf][q0]);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(&sDl[buf][q0 + 4]);
        const float lv[8] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
        const float dl[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
        bool ok[8];
        if (cls == kPartial) {
          const int4 p0 = *reinterpret_cast<const int4*>(&sQp[buf][q0]);
          const int4 p1 = *reinterpret_cast<const int4*>(&sQp[buf][q0 + 4]);
          const int4 o0 = *reinterpret_cast<const int4*>(&sQl[buf][q0]);
          const int4 o1 = *reinterpret_cast<const int4*>(&sQl[buf][q0 + 4]);
          const int qpv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
          const int qlv[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
#pragma unroll
          for (int j = 0; j < 8; ++j) ok[j] = kp >= qlv[j] && kp <= qpv[j];
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) ok[j] = true;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 8 * gg + j;
          const float pr = ok[j] ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], p.c2, -lv[j])) : 0.f;
          const float ds = pr * (dp[r] - dl[j]);
          pb[gg][j] = (__bf16)pr;
          db[gg][j] = (__bf16)ds;
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over this sub-tile's 32 query rows
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int kg = 2 * sub + gg;
#pragma unroll
        for (int t = 0; t < C::DT; ++t) {
          const bf16x8 ao = *reinterpret_cast<const bf16x8*>(dot_t + taddr[kg] + t * 32 * C::TROW);
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(qt_t + taddr[kg] + t * 32 * C::TROW);
          dva[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, pb[gg], dva[t], 0, 0, 0);
          dka[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, db[gg], dka[t], 0, 0, 0);
        }
      }
    }
  };

  const int total = g * p.nqt;
  const int csh = 2 * wave;
  for (int u0 = 0; u0 < total; u0 += C::LIST) {
    const int cnt = build(u0, min(total, u0 + C::LIST));
    if (cnt == 0) continue;
    issue(0, __builtin_amdgcn_readfirstlane(sList[0].x));
    wait_vmem();
    __syncthreads();
    for (int j = 0; j < cnt; ++j) {
      const int cur = j & 1;
      if (j + 1 < cnt) issue(cur ^ 1, __builtin_amdgcn_readfirstlane(sList[j + 1].x));
      compute(cur, (int)(((unsigned)__builtin_amdgcn_readfirstlane(sList[j].y) >> csh) & 3));
      wait_vmem();
      __syncthreads();
    }
  }

  // ---- accumulate into dK, dV (this lane's key; d = 32t + 8*(r/4) + 4*hi + r%4)
  if (kvalid) {
    float* dkr = p.dk + (((long long)b * p.Hkv + kvh) * p.sk + krow) * D;
    float* dvr = p.dv + (((long long)b * p.Hkv + kvh) * p.sk + krow) * D;
#pragma unroll
    for (int t = 0; t < C::DT; ++t)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int dd = 32 * t + 8 * rg + 4 * hi;
        f32x4 k4 = *reinterpret_cast<f32x4*>(dkr + dd);
        f32x4 v4 = *reinterpret_cast<f32x4*>(dvr + dd);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k4[e] += p.scale * dka[t][4 * rg + e];
          v4[e] += dva[t][4 * rg + e];
        }
        *reinterpret_cast<f32x4*>(dkr + dd) = k4;
        *reinterpret_cast<f32x4*>(dvr + dd) = v4;
      }
  }
#endif
}

// ============================================================================
// dQ
// ============================================================================
template <int D>
struct QCfg {
  static constexpr int NW = 8;
  static constexpr int ROW = D * 2;           // bytes per K / V row in LDS
  static constexpr int CHR = D / 8;
  static constexpr int TROW = kKT * 2;        // bytes per K^T row in LDS (128)
  static constexpr int TCHR = kKT / 8;
  static constexpr int RBYTES = kKT * ROW;
  static constexpr int TBYTES = D * TROW;
  static constexpr int RPW = RBYTES / 1024 / NW;
  static constexpr int TPW = TBYTES / 1024 / NW;
  static constexpr int QREG = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int LIST = 2048;
  static_assert(RPW >= 1 && TPW >= 1, "tile too small for the DMA split");
};

template <int D>
__global__ __launch_bounds__(512, 1) void dq_kernel(BParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = QCfg<D>;
  constexpr int NW = C::NW;
  __shared__ __attribute__((aligned(1024))) char sK[2][C::RBYTES];
  __shared__ __attribute__((aligned(1024))) char sV[2][C::RBYTES];
  __shared__ __attribute__((aligned(1024))) char sKT[2][C::TBYTES];
  __shared__ __attribute__((aligned(16))) int sP[2][kKT];
  __shared__ int2 sList[C::LIST];
  __shared__ int sCnt[NW];
  __shared__ int sWb[NW][4];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int g = p.Hq / p.Hkv;
  const int nqt = (p.sq + NW * 32 - 1) / (NW * 32);

  int logical = xcd_logical_block();
  const int hg = logical % g;
  logical /= g;
  const int qt = nqt - 1 - logical % nqt;
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
  const float lse2 = valid ? p.lse2[bh * p.sq_pad + row] : 0.f;
  const float dl = valid ? p.dlt[bh * p.sq_pad + row] : 0.f;
  {
    const int a = wave_min(valid ? qp : INT_MAX), bb = wave_max(valid ? qp : INT_MIN);
    const int c = wave_min(valid ? ql : INT_MAX), d = wave_max(valid ? ql : INT_MIN);
    if (lane == 0) {
      sWb[wave][0] = a;
      sWb[wave][1] = bb;
      sWb[wave][2] = c;
      sWb[wave][3] = d;
    }
  }
  __syncthreads();

  const long long k_row_bytes = p.k_ss * 2;
  const long long v_row_bytes = p.v_ss * 2;
  const long long t_row_bytes = p.kt_row * 2;
  int voffK[C::RPW], voffV[C::RPW], voffT[C::TPW];
#pragma unroll
  for (int j = 0; j < C::RPW; ++j) {
    const int c = (wave + NW * j) * 64 + lane;
    const int r = c / C::CHR, ph = c % C::CHR;
    voffK[j] = (int)(r * k_row_bytes) + 16 * swz<C::CHR>(r, ph);
    voffV[j] = (int)(r * v_row_bytes) + 16 * swz<C::CHR>(r, ph);
  }
#pragma unroll
  for (int j = 0; j < C::TPW; ++j) {
    const int c = (wave + NW * j) * 64 + lane;
    const int r = c / C::TCHR, ph = c % C::TCHR;
    voffT[j] = (int)(r * t_row_bytes) + 16 * swz<C::TCHR>(r, ph);
  }
  const int krow = key_perm(l32);
  int raddr[C::QREG];
#pragma unroll
  for (int kk = 0; kk < C::QREG; ++kk) raddr[kk] = krow * C::ROW + 16 * swz<C::CHR>(krow, 2 * kk + hi);
  int taddr[4];
#pragma unroll
  for (int kg = 0; kg < 4; ++kg) taddr[kg] = l32 * C::TROW + 16 * swz<C::TCHR>(l32, 2 * kg + hi);

  const char* kbase = p.k + ((long long)b * p.k_sb + (long long)kvh * p.k_sh) * 2;
  const char* vbase = p.v + ((long long)b * p.v_sb + (long long)kvh * p.v_sh) * 2;
  const char* ktbase = p.kt + (((long long)b * p.Hkv + kvh) * D) * p.kt_row * 2;
  const __amdgpu_buffer_rsrc_t rsT =
      __builtin_amdgcn_make_buffer_rsrc((void*)ktbase, 0, (int)(D * t_row_bytes), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsP = __builtin_amdgcn_make_buffer_rsrc((void*)p.kpos_pad, 0, 0x7fffffff, kBufferFlags);

  auto issue = [&](int buf, int e) __attribute__((always_inline)) {
    const int src = e & 0xFF, i = (e >> 8) & 0xFFFF;
    const int tile = src * p.tpr + i;
    const int r0 = src * p.R + i * kKT;
    const int nval = min(kKT, p.R - i * kKT);
    const __amdgpu_buffer_rsrc_t rsK = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kbase + (long long)r0 * k_row_bytes), 0, (int)(nval * k_row_bytes), kBufferFlags);
    const __amdgpu_buffer_rsrc_t rsV = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vbase + (long long)r0 * v_row_bytes), 0, (int)(nval * v_row_bytes), kBufferFlags);
#pragma unroll
    for (int j = 0; j < C::RPW; ++j) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsK, (lds_ptr_t)(&sK[buf][0] + (wave + NW * j) * 1024), 16, voffK[j], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsV, (lds_ptr_t)(&sV[buf][0] + (wave + NW * j) * 1024), 16, voffV[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < C::TPW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsT, (lds_ptr_t)(&sKT[buf][0] + (wave + NW * j) * 1024), 16, voffT[j],
                                               tile * kKT * 2, 0, 0);
    if (wave == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsP, (lds_ptr_t)&sP[buf][0], 4, lane * 4, tile * kKT * 4, 0, 0);
  };

  f32x16 dqa[C::DT];
#pragma unroll
  for (int t = 0; t < C::DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[t][r] = 0.f;

  auto compute = [&](int buf, int cls) __attribute__((always_inline)) {
    if (cls == kSkip) return;
    const char* k_t = &sK[buf][0];
    const char* v_t = &sV[buf][0];
    const char* kt_t = &sKT[buf][0];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      // S^T = K Q^T, dP^T = V dO^T for 32 keys (register r: key 32*sub + 16*(r/8) + 8*hi + r%8)
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int kk = 0; kk < C::QREG; ++kk) {
        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(k_t + raddr[kk] + sub * 32 * C::ROW);
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(v_t + raddr[kk] + sub * 32 * C::ROW);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qreg[kk], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, oreg[kk], dp, 0, 0, 0);
      }
      bf16x8 db[2];
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        bool ok[8];
        if (cls == kPartial) {
          const int* kpp = &sP[buf][32 * sub + 16 * gg + 8 * hi];
          const int4 k0 = *reinterpret_cast<const int4*>(kpp);
          const int4 k1 = *reinterpret_cast<const int4*>(kpp + 4);
          const int kv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
          for (int j = 0; j < 8; ++j) ok[j] = kv[j] >= ql && kv[j] <= qp;
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) ok[j] = true;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 8 * gg + j;
          const float pr = ok[j] ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], p.c2, -lse2)) : 0.f;
          db[gg][j] = (__bf16)(pr * (dp[r] - dl));
        }
      }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int kg = 2 * sub + gg;
#pragma unroll
        for (int t = 0; t < C::DT; ++t) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt_t + taddr[kg] + t * 32 * C::TROW);
          dqa[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, db[gg], dqa[t], 0, 0, 0);
        }
      }
    }
  };

  const int total = p.cp * p.tpr;
  const int csh = 2 * wave;
  for (int u0 = 0; u0 < total; u0 += C::LIST) {
    const int cnt = build_key_list<kKT, NW>(p.kbounds, p.tpr, p.rank, p.cp, u0, min(total, u0 + C::LIST), tid, wave,
                                            lane, sWb, sList, sCnt);
    if (cnt == 0) continue;
    issue(0, __builtin_amdgcn_readfirstlane(sList[0].x));
    wait_vmem();
    __syncthreads();
    for (int j = 0; j < cnt; ++j) {
      const int cur = j & 1;
      if (j + 1 < cnt) issue(cur ^ 1, __builtin_amdgcn_readfirstlane(sList[j + 1].x));
      compute(cur, (int)(((unsigned)__builtin_amdgcn_readfirstlane(sList[j].y) >> csh) & 3));
      wait_vmem();
      __syncthreads();
    }
  }

  if (valid) {
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
  p.kt = ws + w.kt_off;
  p.qbounds = reinterpret_cast<const int4*>(ws + w.qbounds_off);
  p.qpos_pad = reinterpret_cast<const int*>(ws + w.qpos_off);
  p.qlo_pad = reinterpret_cast<const int*>(ws + w.qlo_off);
  p.lse2 = reinterpret_cast<const float*>(ws + w.lse2_off);
  p.dlt = reinterpret_cast<const float*>(ws + w.dlt_off);
  p.qt = ws + w.qt_off;
  p.dot = ws + w.dot_off;
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
  p.kt_row = w.kt_row;
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
    hipLaunchKernelGGL((key_prep_kernel<D>), dim3(ntiles, a.b * a.hkv), dim3(256), 0, stream, p,
                       reinterpret_cast<int4*>(ws + w.kbounds_off), reinterpret_cast<int*>(ws + w.kpos_off),
                       reinterpret_cast<__bf16*>(ws + w.kt_off));
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((query_prep_kernel<D>), dim3(p.nqt, a.b * a.hq), dim3(256), 0, stream, p, a.lse, a.delta,
                     reinterpret_cast<int4*>(ws + w.qbounds_off), reinterpret_cast<int*>(ws + w.qpos_off),
                     reinterpret_cast<int*>(ws + w.qlo_off), reinterpret_cast<float*>(ws + w.lse2_off),
                     reinterpret_cast<float*>(ws + w.dlt_off), reinterpret_cast<__bf16*>(ws + w.qt_off),
                     reinterpret_cast<__bf16*>(ws + w.dot_off));
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (ntiles == 0) return hipSuccess;
  const int t128 = (a.rows_per_rank + 127) / 128;
  const long long nkv = (long long)a.cp * t128 * a.hkv * a.b;
  hipLaunchKernelGGL((dkdv_kernel<D>), dim3((unsigned)nkv), dim3(256), 0, stream, p);
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
  const long long nblk = (rows * 32 + 255) / 256;
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
