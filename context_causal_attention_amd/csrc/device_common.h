// Device-side helpers shared by the forward and backward attention kernels
// (gfx950): vector types, LDS swizzles, the key-order permutation of the MFMA
// accumulator rows, wave reductions, the XCD-aware block remap and the
// ring-ordered key-tile list.
#pragma once

#include <hip/hip_runtime.h>

#include <climits>

namespace cpattn {
namespace dev {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x2 __attribute__((__vector_size__(2 * sizeof(float))));
typedef unsigned int u32x4 __attribute__((__vector_size__(4 * sizeof(unsigned int))));
typedef unsigned int u32x2 __attribute__((__vector_size__(2 * sizeof(unsigned int))));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kInvalidKey = INT_MAX;      // position given to padding keys: never allowed
constexpr int kBufferFlags = 0x00020000;  // buffer descriptor word 3 for gfx9: 32-bit data format
constexpr int kSkip = 0, kPartial = 1, kFull = 2;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

// 16-byte-chunk XOR swizzle of an LDS row of C chunks, chosen so that 16 lanes
// reading the same logical chunk of 16 consecutive rows hit 16 distinct
// positions of a 256-byte bank line.
template <int C>
__device__ __forceinline__ int swz(int row, int chunk) {
  if constexpr (C >= 16) return chunk ^ (row & 15);
  else return chunk ^ ((row >> 1) & 7);
}

// Swizzle for tiles that are read both along rows (ds_read_b128 of 16 lanes
// covering 16 consecutive rows at one chunk) and transposed (ds_read_b64_tr_b16:
// each 16-lane group covers 4 consecutive rows x 4 consecutive chunks).  Rows
// r..r+3 land in four different aligned groups of four chunks, and 16
// consecutive rows at one chunk in 16 different chunks (C = 16) or in the two
// 128-byte halves times 8 chunks (C = 8), so both patterns are conflict free.
template <int C>
__device__ __forceinline__ int swz_t(int row, int chunk) {
  if constexpr (C >= 16) return chunk ^ (((row & 3) << 2) | ((row >> 2) & 3));
  else return chunk ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane l receives element
// l % 4 of the 8-byte reads of lanes l / 4 + 4j, j = 0..3.  If lane s of the
// group reads row k0 + s / 4 at column n0 + 4 (s % 4), lane l therefore gets
// column n0 + l at rows k0..k0+3: the k-major layout of an MFMA operand read
// from a row-major tile whose rows run along k.
// Address arithmetic on LDS-space pointers lets the compiler fold constant
// offsets into the DS instructions' offset field.
typedef __attribute__((address_space(3))) char lds_char;
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
__device__ __forceinline__ lds_char* to_lds(void* p) { return (lds_char*)p; }
__device__ __forceinline__ bf16x8 lds_read8(const lds_char* p) {
  return *(const __attribute__((address_space(3))) bf16x8*)p;
}
__device__ __forceinline__ bf16x8 lds_read_tr(const lds_char* lo, const lds_char* hi) {
  typedef __attribute__((address_space(3))) bf16x4* lp;
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lp)(lo));
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lp)(hi));
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Row order of a 32x32 MFMA operand that makes each lane's 8 consecutive
// accumulator registers cover 8 consecutive rows: bits 2 and 3 of the row
// index swapped.  With the 32x32 accumulator layout (register r of lane half h
// holds row 8*(r/4) + 4*h + r%4), register r then holds row 16*(r/8) + 8*h + r%8.
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

// Sorts x ascending over lanes 0..N-1 of each aligned group of N lanes (a
// bitonic network over lane exchanges; N a power of two, at most 64).
template <int N>
__device__ __forceinline__ int wave_sort(int x, int lane) {
#pragma unroll
  for (int k = 2; k <= N; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int y = __shfl_xor(x, j);
      const bool up = (lane & k) == 0, low = (lane & j) == 0;
      x = (up == low) ? min(x, y) : max(x, y);
    }
  return x;
}

// Largest gap between consecutive values of xs, sorted ascending over lanes
// 0..n-1 (n <= 64): {the value before it, the value after it}, or {INT_MAX,
// INT_MIN} when no two consecutive values are more than one apart.  Every
// lane of the wave returns the same pair.
__device__ __forceinline__ int2 largest_gap(int xs, int n, int lane) {
  const int nxt = __shfl_down(xs, 1);
  const int gap = lane + 1 < n ? nxt - xs : 0;
  const int gmax = wave_max(gap);
  if (gmax <= 1) return int2{INT_MAX, INT_MIN};
  const unsigned long long at = __ballot(lane + 1 < n && gap == gmax);
  const int idx = __builtin_ctzll(at);
  return int2{__shfl(xs, idx), __shfl(nxt, idx)};
}

// Widest hole in the union of the intervals [lo, pos] of the lanes 0..n-1
// with ok set, looked for between the intervals of adjacent lanes (rows in
// position order): {h_lo, h_hi} such that no interval meets any k with h_lo <
// k < h_hi, or {INT_MAX, INT_MIN} when there is none.  The candidate is
// checked against every interval, so rows in any order give a correct (maybe
// empty) answer.  Every lane returns the same pair.
__device__ __forceinline__ int2 interval_hole(int lo, int pos, bool ok, int lane, int n) {
  const int nlo = __shfl_down(lo, 1);
  const int nok = __shfl_down(ok ? 1 : 0, 1);
  const bool cand = lane + 1 < n && ok && nok && nlo > pos;
  const int width = cand ? nlo - pos : 0;
  const int wmax = wave_max(width);
  if (wmax <= 1) return int2{INT_MAX, INT_MIN};
  const int idx = __builtin_ctzll(__ballot(cand && width == wmax));
  const int hlo = __shfl(pos, idx), hhi = __shfl(nlo, idx);
  if (__ballot(lane < n && ok && lo < hhi && pos > hlo)) return int2{INT_MAX, INT_MIN};
  return int2{hlo, hhi};
}

// Row bounds of a wave's 32 rows (lanes l and l + 32 hold the same row):
// sWb[wave] = {min q_pos, max q_pos, min q_lo, max q_lo, hole lo, hole hi}.
__device__ __forceinline__ void wave_row_bounds(int wave, int lane, bool valid, int qp, int ql, int (*sWb)[6]) {
  const int a = wave_min(valid ? qp : INT_MAX);
  const int b = wave_max(valid ? qp : INT_MIN);
  const int c = wave_min(valid ? ql : INT_MAX);
  const int d = wave_max(valid ? ql : INT_MIN);
  const int2 h = interval_hole(ql, qp, valid, lane, 32);
  if (lane == 0) {
    sWb[wave][0] = a;
    sWb[wave][1] = b;
    sWb[wave][2] = c;
    sWb[wave][3] = d;
    sWb[wave][4] = h.x;
    sWb[wave][5] = h.y;
  }
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Workgroups are dealt round-robin over the 8 XCDs; this gives each XCD a
// contiguous range of logical ids (neighbouring ids share K/V, hence L2).
__device__ __forceinline__ int xcd_logical_block() {
  const int nblk = gridDim.x;
  const int bid = blockIdx.x;
  const int per_xcd = nblk / 8;
  return bid < per_xcd * 8 ? (bid % 8) * per_xcd + bid / 8 : bid;
}

// Lists, in ring order, the key tiles of schedule slots [u0, u1) that some wave
// of this workgroup needs (u1 - u0 <= CAP).  Slot u is ring step u / tpr (rank
// (rank - step) mod cp) and tile u % tpr of that rank's shard (R rows a
// shard).  Entry .x = src | i << 8; .y = class(wave w) << 2w, from the tile
// bounds {min pos, max pos, gap lo, gap hi} (no key of the tile lies strictly
// between gap lo and gap hi) and each wave's row bounds sWb[w]
// (wave_row_bounds): skip when no key can lie in [min q_lo, max q_pos] outside
// the rows' hole, full when every key lies in [max q_lo, min q_pos] and the
// tile is whole.  Thread t classifies slots u0 + t*PER .. + PER-1 with all its
// bound loads in flight at once, and one prefix sum over the workgroup places
// the active entries: one load latency and two barriers per pass.
template <int BN, int NW, int CAP>
__device__ __forceinline__ int build_key_list(const int4* bounds, int tpr, int R, int rank, int cp, int u0, int u1,
                                              int tid, int wave, int lane, const int (*sWb)[6], int2* sList,
                                              int* sCnt) {
  constexpr int PER = CAP / (NW * 64);
  static_assert(PER >= 1 && PER < 8 && CAP % (NW * 64) == 0, "slots per thread");
  int4 bd[PER];
  int tile_src[PER], tile_i[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int u = min(u0 + tid * PER + j, u1 - 1);
    const int t = u / tpr;
    tile_i[j] = u - t * tpr;
    int src = rank - t;
    if (src < 0) src += cp;
    tile_src[j] = src;
    bd[j] = bounds[src * tpr + tile_i[j]];
  }
  int2 ent[PER];
  int c = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const bool in = u0 + tid * PER + j < u1;
    const bool whole = R - tile_i[j] * BN >= BN;
    unsigned cls_bits = 0;
    bool act = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      int cls = kSkip;
      if (bd[j].x <= sWb[w][1] && bd[j].y >= sWb[w][2] && !(bd[j].z < sWb[w][2] && sWb[w][1] < bd[j].w) &&
          !(sWb[w][4] < bd[j].x && bd[j].y < sWb[w][5]))
        cls = (whole && bd[j].y <= sWb[w][0] && bd[j].x >= sWb[w][3]) ? kFull : kPartial;
      cls_bits |= (unsigned)cls << (2 * w);
      act |= cls != kSkip;
    }
    act = act && in;
    // .x stays below 2^24 (src < 256, tile < 65536): the sign bit marks an
    // entry no wave needs
    ent[j] = int2{tile_src[j] | (tile_i[j] << 8) | (act ? 0 : (int)0x80000000), (int)cls_bits};
    c += act ? 1 : 0;
  }
  // Exclusive prefix of c over the wave from the ballots of its bits (c < 8).
  const unsigned long long lt = (1ull << lane) - 1ull;
  int before = 0, wtot = 0;
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    const unsigned long long m = __ballot((c >> b) & 1);
    before += __popcll(m & lt) << b;
    wtot += __popcll(m) << b;
  }
  if (lane == 0) sCnt[wave] = wtot;
  __syncthreads();
  int off = before, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    off += w < wave ? sCnt[w] : 0;
    tot += sCnt[w];
  }
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (ent[j].x >= 0) sList[off++] = ent[j];
  __syncthreads();
  return tot;
}

}  // namespace dev
}  // namespace cpattn
