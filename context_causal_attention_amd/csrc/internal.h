// Internal declarations shared by the host layer (api.cpp, index.cpp) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <cstdint>
#include <cstddef>

#include <hip/hip_runtime_api.h>

#include "cpattn.h"

namespace cpattn {

// Records a message for cp_last_error() and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Key-tile geometry of the forward kernels: keys are processed in tiles of
// kTileKeys rows that never straddle two ranks' shards.
constexpr int kTileKeysBf16 = 64;
constexpr int kTileKeysF32 = 32;

inline int tile_keys(int32_t dtype) { return dtype == CP_BF16 ? kTileKeysBf16 : kTileKeysF32; }

// bf16 rings of at least this many keys may take the forward's wide launch,
// which reads a transposed copy of V kept in the workspace (when the call has
// no document masks); shorter ones read V in place.
constexpr int64_t kFwdWideKeys = 65536;
inline bool fwd_wide_keys(int32_t dtype, int64_t sk) { return dtype == CP_BF16 && sk >= kFwdWideKeys; }

// Everything the forward launch needs, resolved and validated on the host.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* q_pos;
  const int32_t* q_lo;  // may be null
  const int32_t* k_pos;
  void* o;
  float* lse;
  int64_t q_str[3], k_str[3], v_str[3], o_str[3];
  int32_t b, hq, hkv, d;
  int32_t sq;
  int32_t sk;
  int32_t cp, rank;
  int32_t rows_per_rank;   // sk / cp
  int32_t tiles_per_rank;  // ceil(rows_per_rank / tile_keys)
  float scale_log2;        // scale * log2(e)
  int32_t in_dtype;
  int32_t out_dtype;       // dtype of o (CP_F32 for partial outputs)
  void* ws;                // workspace (layout: see fwd_workspace_layout)
  int32_t merge_acc;       // 1: merge the result into (o, lse) instead of writing it
  int32_t v_in_place;      // 1: never read the transposed copy of V (the workspace holds only the tables)
  int32_t pre_lists;       // 1: the workspace holds the per-query-tile key lists (list_off)
};

struct FwdWorkspace {
  size_t bounds_off;   // int4 per key tile: {min pos, max pos, widest gap lo, gap hi}
  size_t kpos_off;     // int32 per key slot of every tile, padding slots = INT32_MAX (bf16 inputs only)
  size_t order_off;    // int32 per 128-row query tile: listed key tiles, then the dispatch order of
                       // document-masked bf16 launches (bf16 inputs only)
  size_t list_off;     // u32 per (128-row query tile, ring key tile): the key tiles each query tile of a
                       // document-masked bf16 launch lists (fwd_pre_lists shapes only; up to vt_off)
  size_t vt_off;       // bf16 V^T [b][hkv][d][vt_row] (wide bf16 rings only, see fwd_wide_keys)
  size_t total;
  int64_t vt_row;      // elements per V^T row: every key slot of the padded tiles
};

FwdWorkspace fwd_workspace_layout(int32_t b, int32_t hkv, int32_t d, int64_t sq, int64_t sk, int32_t cp,
                                  int32_t in_dtype);
// Query tiles of the document-masked bf16 launch (4 waves of 32 rows), and
// the most of them whose dispatch order is sorted (one workgroup sorts them).
constexpr int kOrderRows = 128;
constexpr int kOrderMaxTiles = 4096;
// Document-masked bf16 launches of at most this many ring key tiles list each
// query tile's key tiles once, in the ordering pass, for all heads.
constexpr int kPreListMaxTiles = 1024;
inline bool fwd_pre_lists(int32_t in_dtype, int64_t sq, int64_t sk, int32_t cp) {
  if (in_dtype != CP_BF16 || cp < 1 || sk <= 0) return false;
  const int64_t n_order = (sq + kOrderRows - 1) / kOrderRows;
  const int64_t ntiles = (sk / cp + kTileKeysBf16 - 1) / kTileKeysBf16 * cp;
  return n_order > 1 && n_order <= kOrderMaxTiles && ntiles <= kPreListMaxTiles;
}

// The allocation-free forward keeps its tile tables (bounds and padded key
// positions, the workspace without the V^T copy) in a static device array of
// this many bytes, one per device (attn_fwd.hip).
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
// This device's address of that array (resolved once per device with
// hipGetSymbolAddress); no allocation.
hipError_t fwd_noalloc_scratch(void** ptr);

// Everything the backward launches need, resolved and validated on the host.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;        // same strides as q
  const void* o;           // final output (delta only), dtype out_dtype, strides o_str
  const int32_t* q_pos;
  const int32_t* q_lo;     // may be null
  const int32_t* k_pos;
  const float* lse;        // [b, hq, sq] contiguous
  const float* delta;      // [b, hq, sq] contiguous
  float* delta_out;        // delta kernel output
  float* dq;               // [b, hq, sq, d] contiguous fp32, accumulated
  float* dk;               // [b, hkv, sk, d] contiguous fp32, accumulated
  float* dv;
  int64_t q_str[3], k_str[3], v_str[3], o_str[3];
  int32_t b, hq, hkv, d;
  int32_t sq, sk;
  int32_t cp, rank;
  int32_t rows_per_rank;   // sk / cp
  float scale;
  int32_t out_dtype;
  void* ws;
};

// Backward key tiles and query tiles both have 64 rows.
constexpr int kBwdTile = 64;

struct BwdWorkspace {
  size_t kbounds_off;  // int4 per key tile: {min pos, max pos, valid rows, 0}
  size_t kpos_off;     // int32 per key slot, padding = INT32_MAX
  size_t qbounds_off;  // int4 per query tile: {min pos, max pos, min lo, max lo}
  size_t qholes_off;   // int2 per query tile: widest hole in the union of its rows' [lo, pos]
  size_t qlo_off;      // int32 [sq_pad]: document start, padding = INT32_MIN
  size_t qspan_off;    // int32 [sq_pad]: position - document start, padding = 0
  size_t nl2_off;      // fp32 [b][hq][sq_pad]: -LSE * log2(e)
  size_t dlt_off;      // fp32 [b][hq][sq_pad]: delta
  size_t kvcost_off;   // int32 per 256-key group of the ring: query tiles listed, then the groups'
                       // dispatch order (bwd_kv_order shapes only)
  size_t qcost_off;    // int32 per 256-row query tile: key tiles listed, then the dQ kernel's dispatch
                       // order under document masks (bwd_q_order shapes only)
  size_t total;
  int64_t kt_row;      // key slots: cp * ceil((sk / cp) / 64) * 64
  int64_t sq_pad;      // ceil(sq / 64) * 64
};

// Backward launches sort the dK/dV kernel's key groups (256 keys of a shard)
// by listed query tiles, most first, when there are 2..kOrderMaxTiles of
// them, and, under document masks, the dQ kernel's 256-row query tiles by
// listed key tiles.
inline int64_t bwd_kv_groups(int64_t sk, int32_t cp) { return cp < 1 ? 0 : (sk / cp + 255) / 256 * cp; }
inline bool bwd_kv_order(int64_t sk, int32_t cp) {
  const int64_t n = bwd_kv_groups(sk, cp);
  return n > 1 && n <= kOrderMaxTiles;
}
inline bool bwd_q_order(int64_t sq) {
  const int64_t n = (sq + 255) / 256;
  return n > 1 && n <= kOrderMaxTiles;
}

BwdWorkspace bwd_workspace_layout(int32_t b, int32_t hq, int32_t hkv, int32_t d, int64_t sq, int64_t sk,
                                  int32_t cp);

// Workgroups of 256 threads for a grid-stride loop over `items` work items:
// enough for one item per thread up to 2^30 items, never more than 2^22
// workgroups, so the grid's work-item count (a 32-bit quantity) stays below
// 2^32 for every size; kernels loop over the rest.
constexpr int64_t kStrideMaxBlocks = (int64_t)1 << 22;
inline unsigned stride_blocks(int64_t items) {
  const int64_t n = items <= 0 ? 0 : (items + 255) / 256;
  return (unsigned)(n < kStrideMaxBlocks ? n : kStrideMaxBlocks);
}

// Kernel launchers (attn_fwd.hip, attn_bwd.hip, merge.hip).  Return hipError_t codes.
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
hipError_t launch_delta(const BwdArgs& a, hipStream_t stream);
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// Sorts n <= kOrderMaxTiles non-negative costs, most first (ties by index), into
// the index list order (one workgroup; attn_fwd.hip).
hipError_t launch_order_sort(const int* cost, int n, int* order, hipStream_t stream);
// The dQ kernel's dispatch order under document masks: per 256-row query tile
// (8 waves of 32 rows) the number of 64-key ring tiles it lists, by the
// forward's rule over the backward's key-tile bounds, then sorted (q_lo must
// not be null; (sq + 255) / 256 <= kOrderMaxTiles).
hipError_t launch_dq_order(const int* q_pos, const int* q_lo, const int4* kbounds, int sq, int R, int tpr, int rank,
                           int cp, int* cost, int* order, hipStream_t stream);
// Head exchange layout kernels (a2a.hip).  unpack = 0: packed [g][H/g][rows][d]
// against the sequence shard [rows, H, d] with row stride x_row_stride
// (elements); unpack = 1: packed against [H/g][g*rows][d].  to_packed = 1
// copies into the packed layout.
hipError_t launch_a2a(int32_t g, int32_t heads, int64_t rows, int32_t d, int32_t dtype, const void* src, void* dst,
                      int64_t x_row_stride, int32_t unpack, int32_t to_packed, hipStream_t stream);
hipError_t launch_merge(int64_t rows, int32_t d, float* o_acc, float* lse_acc, const float* o_p,
                        const float* lse_p, hipStream_t stream);

}  // namespace cpattn
