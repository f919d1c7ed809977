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
};

struct FwdWorkspace {
  size_t bounds_off;   // int4 per key tile: {min pos, max pos, valid rows, 0}
  size_t kpos_off;     // int32 per key slot of every tile, padding slots = INT32_MAX (bf16 inputs only)
  size_t vt_off;       // bf16 V^T [b][hkv][d][cp * tiles_per_rank * tile_keys] (bf16 inputs only)
  size_t total;
  int64_t vt_row;      // elements per V^T row
};

FwdWorkspace fwd_workspace_layout(int32_t b, int32_t hkv, int32_t d, int64_t sk, int32_t cp,
                                  int32_t in_dtype);

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
  size_t total;
  int64_t kt_row;      // key slots: cp * ceil((sk / cp) / 64) * 64
  int64_t sq_pad;      // ceil(sq / 64) * 64
};

BwdWorkspace bwd_workspace_layout(int32_t b, int32_t hq, int32_t hkv, int32_t d, int64_t sq, int64_t sk,
                                  int32_t cp);

// Kernel launchers (attn_fwd.hip, attn_bwd.hip, merge.hip).  Return hipError_t codes.
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
hipError_t launch_delta(const BwdArgs& a, hipStream_t stream);
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// Head exchange layout kernels (a2a.hip).  unpack = 0: packed [g][H/g][rows][d]
// against the sequence shard [rows, H, d] with row stride x_row_stride
// (elements); unpack = 1: packed against [H/g][g*rows][d].  to_packed = 1
// copies into the packed layout.
hipError_t launch_a2a(int32_t g, int32_t heads, int64_t rows, int32_t d, int32_t dtype, const void* src, void* dst,
                      int64_t x_row_stride, int32_t unpack, int32_t to_packed, hipStream_t stream);
hipError_t launch_merge(int64_t rows, int32_t d, float* o_acc, float* lse_acc, const float* o_p,
                        const float* lse_p, hipStream_t stream);

}  // namespace cpattn
