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
//   A workgroup of 4 wave64s owns 128 query rows of one query head (32 rows a
//   wave) and walks the ring's key tiles in step order.  Key tiles never cross
//   a rank's shard; a tile is skipped, computed without masks ("full") or with
//   the per-element mask q_lo <= k_pos <= q_pos ("partial") from the tile's
//   position bounds, at workgroup granularity for loading and at wave
//   granularity for compute.
//
// Matrix-core mapping (bf16: v_mfma_f32_32x32x16_bf16; fp32: 32x32x2 f32)
//   Scores are computed transposed, S^T = K Q^T, so the accumulator column -- a
//   lane modulo 32 -- is a query row: each lane holds 16 (or 32) scores of its
//   own row and the row max / row sum need only one cross-lane exchange
//   (lane ^ 32).  The K operand rows are loaded in a permuted key order (bits 2
//   and 3 of the row index swapped) so that each lane's 8 consecutive
//   accumulator registers hold 8 consecutive keys; those registers, converted to
//   bf16, are directly the B operand of O^T += V^T P^T, with no trip through
//   LDS.  V is staged transposed ([d][keys]) so the V^T operand is one 16-byte
//   LDS read.  The output accumulator O^T likewise keeps one query row per
//   lane, so the online-softmax rescale is one multiply per register.
#include <hip/hip_runtime.h>

#include <climits>
#include <type_traits>

#include "internal.h"

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef unsigned int u32x4 __attribute__((__vector_size__(4 * sizeof(unsigned int))));
typedef unsigned int u32x2 __attribute__((__vector_size__(2 * sizeof(unsigned int))));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;
constexpr int kBlockM = kWaves * kRowsPerWave;
constexpr int kListCap = 2048;          // active key tiles listed per pass
constexpr float kRescaleLog2 = 8.0f;    // keep a stale running max while scores stay within 2^8 of it
constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kInvalidKey = INT_MAX;    // position given to padding keys: never allowed

struct KParams {
  const char* q;
  const char* k;
  const char* v;            // bf16: V^T in the workspace; fp32: V itself
  const int* q_pos;
  const int* q_lo;          // may be null
  const int* k_pos;
  const int4* bounds;       // per key tile {min pos, max pos, valid rows, 0}
  char* o;
  float* lse;
  long long q_sb, q_sh, q_ss;
  long long k_sb, k_sh, k_ss;
  long long v_sb, v_sh, v_ss;  // fp32 V strides; for bf16 V^T: v_ss = row length, v_sh = d * v_ss
  long long o_sb, o_sh, o_ss;
  int B, Hq, Hkv, sq, sk, cp, rank, R, tpr, n_qtiles, out_bf16;
  float c2;                 // softmax scale * log2(e)
};

// 16-byte-chunk XOR swizzle of an LDS row of C chunks, chosen so that 16 lanes
// reading the same logical chunk of 16 consecutive rows hit 16 distinct
// positions of a 256-byte bank line.
template <int C>
__device__ __forceinline__ int swz(int row, int chunk) {
  if constexpr (C >= 16) return chunk ^ (row & 15);
  else return chunk ^ ((row >> 1) & 7);
}

// Key order of the S^T accumulator rows: bits 2 and 3 of the row index swapped.
__device__ __forceinline__ int key_perm(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = min(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = max(x, __shfl_xor(x, o));
  return x;
}

template <bool BF16, int D>
struct Cfg {
  static constexpr int ESZ = BF16 ? 2 : 4;
  static constexpr int BN = BF16 ? kTileKeysBf16 : kTileKeysF32;  // keys per tile
  static constexpr int NSUB = BN / 32;                             // 32-key S^T sub-tiles
  static constexpr int KCHR = D * ESZ / 16;                        // 16-byte chunks per K row
  static constexpr int K_CHUNKS = BN * KCHR;
  static constexpr int VCHR = BF16 ? BN / 8 : D / 4;               // chunks per V^T row (bf16) / V row (fp32)
  static constexpr int V_CHUNKS = BF16 ? D * VCHR : BN * VCHR;
  static constexpr int KLD = K_CHUNKS / kThreads;                  // staged chunks per thread
  static constexpr int VLD = V_CHUNKS / kThreads;
  static constexpr int QREG = BF16 ? D / 16 : D / 2;               // Q operand registers (vectors)
  static constexpr int DT = D / 32;                                // 32-wide output tiles of O^T
  static_assert(K_CHUNKS % kThreads == 0 && V_CHUNKS % kThreads == 0, "tile not divisible");
};

template <bool BF16, int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(KParams p) {
  using C = Cfg<BF16, D>;
  using QT = typename std::conditional<BF16, bf16x8, float>::type;

  __shared__ __attribute__((aligned(16))) u32x4 sK[2][C::K_CHUNKS];
  __shared__ __attribute__((aligned(16))) u32x4 sV[2][C::V_CHUNKS];
  __shared__ __attribute__((aligned(16))) int sKpos[2][C::BN];
  __shared__ int sList[kListCap];
  __shared__ int sCnt[kWaves];
  __shared__ int sWb[kWaves][4];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- block -> (batch, kv head, query tile, query head) ------------------
  // Workgroups are dealt round-robin over the 8 XCDs; give each XCD a
  // contiguous range of logical ids so that the query heads sharing one K/V
  // head (and the same key tiles) run on the same L2.  Within a range, query
  // tiles run from the last (most keys under a causal mask) to the first.
  const int nblk = gridDim.x;
  const int bid = blockIdx.x;
  const int per_xcd = nblk / 8;
  const int logical = bid < per_xcd * 8 ? (bid % 8) * per_xcd + bid / 8 : bid;
  const int g = p.Hq / p.Hkv;
  const int hg = logical % g;
  int rest = logical / g;
  const int qt = p.n_qtiles - 1 - rest % p.n_qtiles;
  rest /= p.n_qtiles;
  const int kvh = rest % p.Hkv;
  const int b = rest / p.Hkv;
  const int h = kvh * g + hg;

  const int row = qt * kBlockM + wave * kRowsPerWave + l32;
  const bool valid = row < p.sq;

  // ---- query operand in registers -----------------------------------------
  QT qreg[C::QREG];
  {
    const char* qrow = p.q + ((long long)b * p.q_sb + (long long)h * p.q_sh + (long long)row * p.q_ss) * C::ESZ;
    if constexpr (BF16) {
#pragma unroll
      for (int kk = 0; kk < C::QREG; ++kk) {
        u32x4 raw = valid ? *reinterpret_cast<const u32x4*>(qrow + (16 * kk + 8 * hi) * 2) : u32x4{0, 0, 0, 0};
        qreg[kk] = __builtin_bit_cast(bf16x8, raw);
      }
    } else {
#pragma unroll
      for (int j = 0; j < D / 8; ++j) {
        f32x4 raw = valid ? *reinterpret_cast<const f32x4*>(qrow + (hi * (D / 2) + 4 * j) * 4) : f32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) qreg[4 * j + e] = raw[e];
      }
    }
  }
  const int qp = valid ? p.q_pos[row] : -1;
  const int ql = valid ? (p.q_lo ? p.q_lo[row] : 0) : INT_MAX;

  // ---- position bounds of this wave's and this workgroup's rows -----------
  const int wqmin = wave_min(valid ? qp : INT_MAX);
  const int wqmax = wave_max(valid ? qp : INT_MIN);
  const int wlmin = wave_min(valid ? ql : INT_MAX);
  const int wlmax = wave_max(valid ? ql : INT_MIN);
  if (lane == 0) {
    sWb[wave][0] = wqmin;
    sWb[wave][1] = wqmax;
    sWb[wave][2] = wlmin;
    sWb[wave][3] = wlmax;
  }
  __syncthreads();
  int gqmax = INT_MIN, glmin = INT_MAX;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    gqmax = max(gqmax, sWb[w][1]);
    glmin = min(glmin, sWb[w][2]);
  }

  // ---- online softmax state ------------------------------------------------
  f32x16 oacc[C::DT];
#pragma unroll
  for (int t = 0; t < C::DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
  float m_run = -INFINITY;  // running max of scale*log2(e)*s, shared by lanes l and l^32
  float l_run = 0.f;        // this lane's part of the running sum

  const long long kbase = (long long)b * p.k_sb + (long long)kvh * p.k_sh;
  const long long vbase = (long long)b * p.v_sb + (long long)kvh * p.v_sh;

  // Staging registers for the next tile.
  u32x4 kst[C::KLD];
  u32x4 vst[C::VLD];
  int kpst = kInvalidKey;
  int4 bd_next = {0, 0, 0, 0};

  auto stage_load = [&](int tile) {
    const int src = tile / p.tpr;
    const int i = tile - src * p.tpr;
    const int r0 = src * p.R + i * C::BN;  // first key row of the tile
    const int nval = min(C::BN, p.R - i * C::BN);
#pragma unroll
    for (int j = 0; j < C::KLD; ++j) {
      const int c = tid + j * kThreads;
      const int r = c / C::KCHR, ch = c % C::KCHR;
      kst[j] = r < nval ? *reinterpret_cast<const u32x4*>(p.k + ((kbase + (long long)(r0 + r) * p.k_ss) * C::ESZ + ch * 16))
                        : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < C::VLD; ++j) {
      const int c = tid + j * kThreads;
      if constexpr (BF16) {
        const int dv = c / C::VCHR, ch = c % C::VCHR;
        vst[j] = *reinterpret_cast<const u32x4*>(p.v + ((vbase + (long long)dv * p.v_ss + (long long)tile * C::BN) * 2 + ch * 16));
      } else {
        const int r = c / C::VCHR, ch = c % C::VCHR;
        vst[j] = r < nval ? *reinterpret_cast<const u32x4*>(p.v + ((vbase + (long long)(r0 + r) * p.v_ss) * 4 + ch * 16))
                          : u32x4{0, 0, 0, 0};
      }
    }
    if (tid < C::BN) kpst = tid < nval ? p.k_pos[r0 + tid] : kInvalidKey;
    bd_next = p.bounds[tile];
  };

  auto stage_store = [&](int buf) {
#pragma unroll
    for (int j = 0; j < C::KLD; ++j) {
      const int c = tid + j * kThreads;
      const int r = c / C::KCHR, ch = c % C::KCHR;
      sK[buf][r * C::KCHR + swz<C::KCHR>(r, ch)] = kst[j];
    }
#pragma unroll
    for (int j = 0; j < C::VLD; ++j) {
      const int c = tid + j * kThreads;
      if constexpr (BF16) {
        const int dv = c / C::VCHR, ch = c % C::VCHR;
        sV[buf][dv * C::VCHR + swz<C::VCHR>(dv, ch)] = vst[j];
      } else {
        sV[buf][c] = vst[j];
      }
    }
    if (tid < C::BN) sKpos[buf][tid] = kpst;
  };

  auto compute = [&](int buf, int4 bd) {
    // Wave-level class of this tile: skip, full (no mask) or partial.
    if (bd.x > wqmax || bd.y < wlmin) return;
    const bool full = bd.z == C::BN && bd.y <= wqmin && bd.x >= wlmax;

    f32x16 sacc[C::NSUB];
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[sub][r] = 0.f;
      const int krow = 32 * sub + key_perm(l32);
      if constexpr (BF16) {
#pragma unroll
        for (int kk = 0; kk < C::QREG; ++kk) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, sK[buf][krow * C::KCHR + swz<C::KCHR>(krow, 2 * kk + hi)]);
          sacc[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], sacc[sub], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int j = 0; j < D / 8; ++j) {
          const f32x4 a = __builtin_bit_cast(f32x4, sK[buf][krow * C::KCHR + swz<C::KCHR>(krow, hi * (D / 8) + j)]);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sacc[sub] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qreg[4 * j + e], sacc[sub], 0, 0, 0);
        }
      }
    }

    // Register r of sub-tile sub holds key 32*sub + 16*(r/8) + 8*hi + r%8.
    if (!full) {
#pragma unroll
      for (int sub = 0; sub < C::NSUB; ++sub)
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const int* kp = &sKpos[buf][32 * sub + 16 * gg + 8 * hi];
          const int4 k0 = *reinterpret_cast<const int4*>(kp);
          const int4 k1 = *reinterpret_cast<const int4*>(kp + 4);
          const int kv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const bool ok = kv[j] >= ql && kv[j] <= qp;
            sacc[sub][8 * gg + j] = ok ? sacc[sub][8 * gg + j] : -INFINITY;
          }
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[sub][r]);
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
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[sub][r], p.c2, -m_use));
        l_run += e;
        sacc[sub][r] = e;
      }

    // O^T += V^T P^T
    if constexpr (BF16) {
#pragma unroll
      for (int kg = 0; kg < 2 * C::NSUB; ++kg) {
        bf16x8 pb;
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[j] = (__bf16)sacc[kg >> 1][8 * (kg & 1) + j];
#pragma unroll
        for (int t = 0; t < C::DT; ++t) {
          const int vr = 32 * t + l32;
          const bf16x8 a = __builtin_bit_cast(bf16x8, sV[buf][vr * C::VCHR + swz<C::VCHR>(vr, 2 * kg + hi)]);
          oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[t], 0, 0, 0);
        }
      }
    } else {
      const float* vf = reinterpret_cast<const float*>(&sV[buf][0]);
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int key = 16 * (s >> 3) + 8 * hi + (s & 7);
#pragma unroll
        for (int t = 0; t < C::DT; ++t)
          oacc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf[key * D + 32 * t + l32], sacc[0][s], oacc[t], 0, 0, 0);
      }
    }
  };

  // ---- walk the ring: list the active key tiles, then stream them ---------
  const int total = p.cp * p.tpr;
  for (int u0 = 0; u0 < total; u0 += kListCap) {
    const int u1 = min(total, u0 + kListCap);
    int cnt = 0;
    for (int base = u0; base < u1; base += kThreads) {
      const int u = base + tid;
      bool act = false;
      int tile = 0;
      if (u < u1) {
        const int t = u / p.tpr;
        const int i = u - t * p.tpr;
        int src = p.rank - t;
        if (src < 0) src += p.cp;
        tile = src * p.tpr + i;
        const int4 bd = p.bounds[tile];
        act = bd.z > 0 && bd.x <= gqmax && bd.y >= glmin;
      }
      const unsigned long long bal = __ballot(act);
      const int before = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) sCnt[wave] = __popcll(bal);
      __syncthreads();
      int off = cnt, tot = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        off += w < wave ? sCnt[w] : 0;
        tot += sCnt[w];
      }
      if (act) sList[off + before] = tile;
      cnt += tot;
      __syncthreads();
    }
    if (cnt == 0) continue;
    stage_load(sList[0]);
    stage_store(0);
    int4 bd_cur = bd_next;
    __syncthreads();
    for (int j = 0; j < cnt; ++j) {
      const int cur = j & 1;
      const bool has_next = j + 1 < cnt;
      if (has_next) stage_load(sList[j + 1]);
      compute(cur, bd_cur);
      if (has_next) stage_store(cur ^ 1);
      bd_cur = bd_next;
      __syncthreads();
    }
  }

  // ---- epilogue: normalise and store O and LSE ----------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  if (valid) {
    if (hi == 0)
      p.lse[((long long)b * p.Hq + h) * p.sq + row] = empty ? -INFINITY : (m_run + log2f(l_tot)) * kLn2;
    const long long obase = (long long)b * p.o_sb + (long long)h * p.o_sh + (long long)row * p.o_ss;
#pragma unroll
    for (int t = 0; t < C::DT; ++t)
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
}

// Per key tile: position bounds and count of valid rows; for bf16 inputs also
// V transposed into the workspace ([b][kv head][d][tile * BN + key], zero in
// the padding of a shard's last tile) so the kernel above can read V^T rows.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void prep_kernel(const int* __restrict__ k_pos, const char* __restrict__ v,
                                                   long long v_sb, long long v_sh, long long v_ss, int Hkv,
                                                   int R, int tpr, int4* __restrict__ bounds, __bf16* vt,
                                                   long long vt_row) {
  using C = Cfg<BF16, D>;
  const int tile = blockIdx.x;
  const int src = tile / tpr;
  const int i = tile - src * tpr;
  const int r0 = src * R + i * C::BN;
  const int nval = min(C::BN, R - i * C::BN);
  const int tid = threadIdx.x;
  if (blockIdx.y == 0 && tid < 64) {
    const bool ok = tid < nval;
    const int kp = ok ? k_pos[r0 + tid] : 0;
    const int mn = wave_min(ok ? kp : INT_MAX);
    const int mx = wave_max(ok ? kp : INT_MIN);
    if (tid == 0) bounds[tile] = int4{mn, mx, nval, 0};
  }
  if constexpr (BF16) {
    __shared__ __bf16 s[C::BN][D + 8];
    const int b = blockIdx.y / Hkv, kvh = blockIdx.y % Hkv;
    const char* vb = v + ((long long)b * v_sb + (long long)kvh * v_sh) * 2;
    constexpr int CH = D / 8;  // 16-byte chunks per V row
    for (int c = tid; c < C::BN * CH; c += 256) {
      const int r = c / CH, ch = c % CH;
      u32x4 raw = r < nval ? *reinterpret_cast<const u32x4*>(vb + ((long long)(r0 + r) * v_ss + ch * 8) * 2)
                           : u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(&s[r][ch * 8]) = raw;
    }
    __syncthreads();
    __bf16* out = vt + ((long long)blockIdx.y * D) * vt_row + (long long)tile * C::BN;
    for (int c = tid; c < D * (C::BN / 8); c += 256) {
      const int dv = c / (C::BN / 8), kc = c % (C::BN / 8);
      bf16x8 w;
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = s[kc * 8 + j][dv];
      *reinterpret_cast<bf16x8*>(out + (long long)dv * vt_row + kc * 8) = w;
    }
  }
}

template <bool BF16, int D>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  using C = Cfg<BF16, D>;
  const FwdWorkspace w = fwd_workspace_layout(a.b, a.hkv, a.d, a.sk, a.cp, a.in_dtype);
  char* ws = static_cast<char*>(a.ws);
  int4* bounds = reinterpret_cast<int4*>(ws + w.bounds_off);
  __bf16* vt = reinterpret_cast<__bf16*>(ws + w.vt_off);
  const int ntiles = a.cp * a.tiles_per_rank;
  if (ntiles > 0) {
    dim3 grid(ntiles, BF16 ? a.b * a.hkv : 1);
    hipLaunchKernelGGL((prep_kernel<BF16, D>), grid, dim3(256), 0, stream, a.k_pos,
                       static_cast<const char*>(a.v), (long long)a.v_str[0], (long long)a.v_str[1],
                       (long long)a.v_str[2], a.hkv, a.rows_per_rank, a.tiles_per_rank, bounds, vt,
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
  p.n_qtiles = (a.sq + kBlockM - 1) / kBlockM;
  p.out_bf16 = a.out_dtype == CP_BF16;
  p.c2 = a.scale_log2;
  const long long nblk = (long long)p.n_qtiles * a.hq * a.b;
  hipLaunchKernelGGL((fwd_kernel<BF16, D>), dim3((unsigned)nblk), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  if (a.in_dtype == CP_BF16) return a.d == 64 ? launch_t<true, 64>(a, stream) : launch_t<true, 128>(a, stream);
  return a.d == 64 ? launch_t<false, 64>(a, stream) : launch_t<false, 128>(a, stream);
}

}  // namespace cpattn
