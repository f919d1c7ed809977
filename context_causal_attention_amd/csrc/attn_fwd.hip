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
constexpr float kRescaleLog2 = 8.0f;    // keep a stale running max while scores stay within 2^8 of it

struct KParams {
  const char* q;
  const char* k;
  const char* v;            // bf16: V^T in the workspace; fp32: V itself
  const int* q_pos;
  const int* q_lo;          // may be null
  const int* k_pos;
  const int* kpos_pad;      // bf16: key positions per tile slot, padding = kInvalidKey
  const int4* bounds;       // per key tile {min pos, max pos, gap lo, gap hi}
  char* o;
  float* lse;
  long long q_sb, q_sh, q_ss;
  long long k_sb, k_sh, k_ss;
  long long v_sb, v_sh, v_ss;  // fp32 V strides; for bf16 V^T: v_ss = row length, v_sh = d * v_ss
  long long o_sb, o_sh, o_ss;
  int B, Hq, Hkv, sq, sk, cp, rank, R, tpr, n_qtiles, out_bf16;
  int merge_acc;            // 1: (o, lse) hold a partial result over other keys (fp32) to merge into
  float c2;                 // softmax scale * log2(e)
};

// Work item of this workgroup.  Workgroups are dealt round-robin over the 8
// XCDs; each XCD gets a contiguous range of logical ids so that the query heads
// sharing one K/V head (and the same key tiles) run on the same L2.  Within a
// range, query tiles run from the last (most keys under a causal mask) to the
// first.
struct Item {
  int b, h, kvh, qt;
};
__device__ __forceinline__ Item map_block(const KParams& p) {
  const int logical = xcd_logical_block();
  const int g = p.Hq / p.Hkv;
  const int hg = logical % g;
  int rest = logical / g;
  Item it;
  it.qt = p.n_qtiles - 1 - rest % p.n_qtiles;
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

// ============================================================================
// bf16 kernel
// ============================================================================
template <int D, int NW>
struct Bf16Cfg {
  static constexpr int BN = kTileKeysBf16;       // keys per tile
  static constexpr int KROW = D * 2;             // bytes per K row in LDS
  static constexpr int KCHR = D / 8;             // 16-byte chunks per K row
  static constexpr int VROW = BN * 2;            // bytes per V^T row in LDS (128)
  static constexpr int VCHR = BN / 8;            // 8
  static constexpr int KBYTES = BN * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int KPW = KBYTES / 1024 / NW;  // 1 KB DMA blocks per wave
  static constexpr int VPW = VBYTES / 1024 / NW;
  static constexpr int QREG = D / 16;
  static constexpr int DT = D / 32;
  static_assert(KPW >= 1 && VPW >= 1, "tile too small for the DMA split");
};

// NW waves of 32 query rows each; two waves share each SIMD (NW = 8: one
// workgroup per CU; NW = 4: two).
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 8 / NW) void fwd_bf16_kernel(KParams p) {
  // The body uses device-only buffer-descriptor types; the host pass only needs
  // the launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  using C = Bf16Cfg<D, NW>;
  __shared__ __attribute__((aligned(1024))) char sK0[C::KBYTES];
  __shared__ __attribute__((aligned(1024))) char sK1[C::KBYTES];
  __shared__ __attribute__((aligned(1024))) char sV0[C::VBYTES];
  __shared__ __attribute__((aligned(1024))) char sV1[C::VBYTES];
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

  // ---- query operand (B of S^T = K Q^T) in registers ----------------------
  bf16x8 qreg[C::QREG];
  {
    const char* qrow = p.q + ((long long)it.b * p.q_sb + (long long)it.h * p.q_sh + (long long)row * p.q_ss) * 2;
#pragma unroll
    for (int kk = 0; kk < C::QREG; ++kk) {
      const u32x4 raw = valid ? *reinterpret_cast<const u32x4*>(qrow + (16 * kk + 8 * hi) * 2) : u32x4{0, 0, 0, 0};
      qreg[kk] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  const int qp = valid ? p.q_pos[row] : -1;
  const int ql = valid ? (p.q_lo ? p.q_lo[row] : 0) : INT_MAX;
  wave_row_bounds(wave, lane, valid, qp, ql, sWb);
  __syncthreads();

  // ---- per-lane constant addresses ------------------------------------------
  // DMA: this lane's 16-byte slot in each of the wave's 1 KB blocks.
  const long long k_row_bytes = p.k_ss * 2;
  int voffK[C::KPW], voffV[C::VPW];
#pragma unroll
  for (int j = 0; j < C::KPW; ++j) {
    const int c = (wave + NW * j) * 64 + lane;  // physical chunk index within the K tile
    const int r = c / C::KCHR, ph = c % C::KCHR;
    voffK[j] = (int)(r * k_row_bytes) + 16 * swz<C::KCHR>(r, ph);
  }
  const long long vt_row_bytes = p.v_ss * 2;
#pragma unroll
  for (int j = 0; j < C::VPW; ++j) {
    const int c = (wave + NW * j) * 64 + lane;
    const int r = c / C::VCHR, ph = c % C::VCHR;
    voffV[j] = (int)(r * vt_row_bytes) + 16 * swz<C::VCHR>(r, ph);
  }
  // LDS reads: K operand rows key_perm(l32) (+32 for the second sub-tile),
  // V^T operand rows l32 (+32 per output tile).
  const int krow = key_perm(l32);
  int kaddr[C::QREG];
#pragma unroll
  for (int kk = 0; kk < C::QREG; ++kk) kaddr[kk] = krow * C::KROW + 16 * swz<C::KCHR>(krow, 2 * kk + hi);
  int vaddr[4];
#pragma unroll
  for (int kg = 0; kg < 4; ++kg) vaddr[kg] = l32 * C::VROW + 16 * swz<C::VCHR>(l32, 2 * kg + hi);

  const char* kbase = p.k + ((long long)it.b * p.k_sb + (long long)it.kvh * p.k_sh) * 2;
  const char* vtbase = p.v + ((long long)it.b * p.v_sb + (long long)it.kvh * p.v_sh) * 2;
  const __amdgpu_buffer_rsrc_t rsV =
      __builtin_amdgcn_make_buffer_rsrc((void*)vtbase, 0, (int)(D * vt_row_bytes), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsP =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.kpos_pad, 0, 0x7fffffff, kBufferFlags);

  // List entry: src | i << 8 | class(wave w) << (24 + 2w) for key tile i of
  // rank src's shard (tile id src * tpr + i).
  auto tile_of = [&](int e) { return (e & 0xFF) * p.tpr + ((e >> 8) & 0xFFFF); };
  // Copies K of list entry e (uniform) into LDS buffer `buf` (static).
  auto issue_k = [&](auto bufc, int e) {
    constexpr int buf = decltype(bufc)::value;
    char* sK = buf ? sK1 : sK0;
    const int src = e & 0xFF, i = (e >> 8) & 0xFFFF;
    const int r0 = src * p.R + i * C::BN;
    const int nval = min(C::BN, p.R - i * C::BN);
    const __amdgpu_buffer_rsrc_t rsK = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kbase + (long long)r0 * k_row_bytes), 0, (int)(nval * k_row_bytes), kBufferFlags);
#pragma unroll
    for (int j = 0; j < C::KPW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsK, (lds_ptr_t)(sK + (wave + NW * j) * 1024), 16, voffK[j], 0, 0, 0);
  };
  // Copies V^T and the key positions of list entry e into LDS buffer `buf`.
  auto issue_v = [&](auto bufc, int e) {
    constexpr int buf = decltype(bufc)::value;
    char* sV = buf ? sV1 : sV0;
    int* sP = buf ? sP1 : sP0;
    const int tile = tile_of(e);
#pragma unroll
    for (int j = 0; j < C::VPW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsV, (lds_ptr_t)(sV + (wave + NW * j) * 1024), 16, voffV[j],
                                               tile * C::BN * 2, 0, 0);
    if (wave == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsP, (lds_ptr_t)sP, 4, lane * 4, tile * C::BN * 4, 0, 0);
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

  // S^T = K Q^T of the tile in K buffer kb: 16 MFMAs into (s0, s1).
  auto scores = [&](auto kbc, f32x16& s0, f32x16& s1) {
    constexpr int kb = decltype(kbc)::value;
    const char* sK = kb ? sK1 : sK0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = 0.f;
      s1[r] = 0.f;
    }
#pragma unroll
    for (int kk = 0; kk < C::QREG; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + kaddr[kk]);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(sK + kaddr[kk] + 32 * C::KROW);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, qreg[kk], s1, 0, 0, 0);
    }
  };
  // P = exp2(c2*s - m) of group kg (8 keys) rounded to bf16; the fp32 values
  // go into the tile's row sum (the LSE needs them unrounded).
  auto expg = [&](const f32x16& c0, const f32x16& c1, int kg, float nm, bf16x8& pb, float& lj) {
    const f32x16& sv = kg < 2 ? c0 : c1;
    const int base = 8 * (kg & 1);
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[base + j], p.c2, nm));
      const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[base + j + 1], p.c2, nm));
      const bf16x2 pr = __builtin_convertvector((f32x2){e0, e1}, bf16x2);
      lj += e0 + e1;
      pb[j] = pr[0];
      pb[j + 1] = pr[1];
    }
  };

  // One pipeline stage: tile j's scores (c0, c1) are masked, exponentiated
  // and multiplied into O (V^T from buffer vb) while tile j+1's scores are
  // computed into (n0, n1) from K buffer kb.
  auto stage = [&](auto kbc, auto vbc, f32x16& c0, f32x16& c1, f32x16& n0, f32x16& n1, int cls_cur) {
    constexpr int vb = decltype(vbc)::value;
    const char* sV = vb ? sV1 : sV0;
    const int* sP = vb ? sP1 : sP0;
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
    bf16x8 pb[4];
    float lj = 0.f;
    const float nm = -m_run;
    {
      // 16 chunks, fenced from each other: chunk m reads the K operand of MFMA
      // m+4, issues MFMA m of the next tile's scores (sub-tile m%2, d-slice
      // m/2), and exponentiates scores 2m, 2m+1 of this tile.
      constexpr int kb = decltype(kbc)::value;
      const char* sK = kb ? sK1 : sK0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        n0[r] = 0.f;
        n1[r] = 0.f;
      }
      auto kop = [&](int m) {
        return *reinterpret_cast<const bf16x8*>(sK + kaddr[m >> 1] + (m & 1) * 32 * C::KROW);
      };
      // Issue priority 1 for this block, 0 again from the P V MFMAs on: while
      // one wave interleaves scores and exponentials, the SIMD's other wave
      // fills the gaps (1-2% faster than equal priority throughout).
      __builtin_amdgcn_s_setprio(1);
      constexpr int NM = 2 * C::QREG;  // MFMAs per tile
      constexpr int PF = 4;            // operand reads in flight
      bf16x8 ops[NM];
#pragma unroll
      for (int m = 0; m < PF; ++m) ops[m] = kop(m);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
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
    // O^T += V^T P^T
    bf16x8 va[C::DT];
#pragma unroll
    for (int t = 0; t < C::DT; ++t) va[t] = *reinterpret_cast<const bf16x8*>(sV + vaddr[0] + t * 32 * C::VROW);
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
#pragma unroll
      for (int t = 0; t < C::DT; ++t) {
        oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t], pb[kg], oacc[t], 0, 0, 0);
        if (kg < 3) va[t] = *reinterpret_cast<const bf16x8*>(sV + vaddr[kg + 1] + t * 32 * C::VROW);
      }
    }
  };

  // ---- walk the ring: list the needed key tiles, then stream them ---------
  // Iteration j reads K of tile j+1 and V^T of tile j while tile j+2's K and
  // tile j+1's V^T are copied in; buffers alternate, so the loop is unrolled
  // by two with static buffer and register roles.
  f32x16 sa0, sa1, sb0, sb1;
  const int total = p.cp * p.tpr;
  const int csh = 2 * wave;
  auto cls_of = [&](int2 e) { return (int)(((unsigned)e.y >> csh) & 3); };
  for (int u0 = 0; u0 < total; u0 += kListCap) {
    const int cnt = build_key_list<C::BN, NW>(p.bounds, p.tpr, p.R, p.rank, p.cp, u0, min(total, u0 + kListCap), tid,
                                                  wave, lane, sWb, sList, sCnt);
    if (cnt == 0) continue;
    // Entry of list slot j (x: tile, y: classes), read as scalars.
    auto entry = [&](int j) {
      int2 e = {0, 0};
      if (j < cnt) {
        e.x = __builtin_amdgcn_readfirstlane(sList[j].x);
        e.y = __builtin_amdgcn_readfirstlane(sList[j].y);
      }
      return e;
    };
    int2 e_cur = entry(0), e_nxt = entry(1);
    issue_k(std::integral_constant<int, 0>{}, e_cur.x);
    issue_v(std::integral_constant<int, 0>{}, e_cur.x);
    if (cnt > 1) issue_k(std::integral_constant<int, 1>{}, e_nxt.x);
    wait_vmem();
    __syncthreads();
    if (cls_of(e_cur) != kSkip) scores(std::integral_constant<int, 0>{}, sa0, sa1);
    __syncthreads();
    for (int j = 0;;) {
      // K of tile j+1 in buffer 1, V^T of tile j in buffer 0; scores of tile j in sa.
      {
        const int2 e2 = entry(j + 2);
        if (j + 2 < cnt) issue_k(std::integral_constant<int, 0>{}, e2.x);
        if (j + 1 < cnt) issue_v(std::integral_constant<int, 1>{}, e_nxt.x);
        stage(std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{}, sa0, sa1, sb0, sb1, cls_of(e_cur));
        wait_vmem();
        __syncthreads();
        e_cur = e_nxt;
        e_nxt = e2;
      }
      if (++j >= cnt) break;
      // K of tile j+1 in buffer 0, V^T of tile j in buffer 1; scores of tile j in sb.
      {
        const int2 e2 = entry(j + 2);
        if (j + 2 < cnt) issue_k(std::integral_constant<int, 1>{}, e2.x);
        if (j + 1 < cnt) issue_v(std::integral_constant<int, 0>{}, e_nxt.x);
        stage(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}, sb0, sb1, sa0, sa1, cls_of(e_cur));
        wait_vmem();
        __syncthreads();
        e_cur = e_nxt;
        e_nxt = e2;
      }
      if (++j >= cnt) break;
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (valid) store_out<C::DT>(p, it, row, hi, m_run, l_tot, oacc);
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
    const int cnt = build_key_list<C::BN, kF32Waves>(p.bounds, p.tpr, p.R, p.rank, p.cp, u0, min(total, u0 + kListCap), tid,
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

// Per key tile: position bounds and count of valid rows.  For bf16 inputs also
// the key positions padded per tile slot and V transposed into the workspace
// ([b][kv head][d][tile * BN + key], zero in the padding of a shard's last
// tile) so the kernel above can read V^T rows.
template <bool BF16, int D>
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
  if constexpr (BF16) {
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

template <bool BF16, int D>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  const FwdWorkspace w = fwd_workspace_layout(a.b, a.hkv, a.d, a.sk, a.cp, a.in_dtype);
  char* ws = static_cast<char*>(a.ws);
  int4* bounds = reinterpret_cast<int4*>(ws + w.bounds_off);
  int* kpos_pad = reinterpret_cast<int*>(ws + w.kpos_off);
  __bf16* vt = reinterpret_cast<__bf16*>(ws + w.vt_off);
  const int ntiles = a.cp * a.tiles_per_rank;
  if (ntiles > 0) {
    dim3 grid(ntiles, BF16 ? a.b * a.hkv : 1);
    hipLaunchKernelGGL((prep_kernel<BF16, D>), grid, dim3(256), 0, stream, a.k_pos,
                       static_cast<const char*>(a.v), (long long)a.v_str[0], (long long)a.v_str[1],
                       (long long)a.v_str[2], a.hkv, a.rows_per_rank, a.tiles_per_rank, bounds, kpos_pad, vt,
                       (long long)w.vt_row);
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
  p.o = static_cast<char*>(a.o);
  p.lse = a.lse;
  p.q_sb = a.q_str[0];
  p.q_sh = a.q_str[1];
  p.q_ss = a.q_str[2];
  p.k_sb = a.k_str[0];
  p.k_sh = a.k_str[1];
  p.k_ss = a.k_str[2];
  if constexpr (BF16) {
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
    // Wave count of the bf16 kernel (results are the same bits either way):
    // 8 waves share each K/V tile copy, the better choice when every row sees
    // many keys (dense causal rings of >= 65536 keys, 1% faster at 131072);
    // two 4-wave workgroups per CU keep their barriers apart, better for
    // shorter rings (1.5% at 32768 keys) and for document masks, whose rows
    // see few keys (4-10%).
    const bool wide = a.q_lo == nullptr && a.sk >= 65536;
    const int nw = wide ? 8 : 4;
    p.n_qtiles = (a.sq + nw * kRowsPerWave - 1) / (nw * kRowsPerWave);
    const long long nblk = (long long)p.n_qtiles * a.hq * a.b;
    if (wide)
      hipLaunchKernelGGL((fwd_bf16_kernel<D, 8>), dim3((unsigned)nblk), dim3(8 * 64), 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<D, 4>), dim3((unsigned)nblk), dim3(4 * 64), 0, stream, p);
  } else {
    p.n_qtiles = (a.sq + kF32BlockM - 1) / kF32BlockM;
    const long long nblk = (long long)p.n_qtiles * a.hq * a.b;
    hipLaunchKernelGGL((fwd_f32_kernel<D>), dim3((unsigned)nblk), dim3(kF32Threads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace fwdk

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  using namespace fwdk;
  if (a.in_dtype == CP_BF16) return a.d == 64 ? launch_t<true, 64>(a, stream) : launch_t<true, 128>(a, stream);
  return a.d == 64 ? launch_t<false, 64>(a, stream) : launch_t<false, 128>(a, stream);
}

}  // namespace cpattn
