// C ABI of libcpattn.so: argument validation, workspace layout and dispatch to
// the HIP kernels.  Every check happens before anything is enqueued, so a call
// that returns an error has launched nothing.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

#include "internal.h"

namespace cpattn {

namespace {
thread_local std::string g_last_error;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int esize(int32_t dtype) { return dtype == CP_BF16 ? 2 : 4; }

int check_dtype(int32_t dt, const char* what) {
  if (dt != CP_F32 && dt != CP_BF16) return fail(CP_EDTYPE, "%s: unknown dtype code %d", what, dt);
  return CP_OK;
}

int check_strides(const int64_t* st, int32_t dtype, const char* what) {
  for (int i = 0; i < 3; ++i) {
    if (st[i] < 0) return fail(CP_EINVAL, "%s stride %d is negative", what, i);
    // Element size 2 or 4 divides 16: a multiple of 16 bytes is a multiple
    // of 16 / esize elements (tested without forming the byte count).
    if (st[i] % (16 / (int64_t)esize(dtype)) != 0)
      return fail(CP_EINVAL, "%s stride %d (%lld elements) is not a multiple of 16 bytes", what, i,
                  (long long)st[i]);
  }
  return CP_OK;
}

// The kernels form element offsets b*sb + h*sh + row*ss in 64-bit integers:
// the largest one, plus a row, must stay below 2^62.
int check_extent(int64_t nb, int64_t nh, int64_t rows, int32_t d, const int64_t* st, const char* what) {
  const double ext = (double)(nb > 0 ? nb - 1 : 0) * (double)st[0] + (double)(nh > 0 ? nh - 1 : 0) * (double)st[1] +
                     (double)(rows > 0 ? rows - 1 : 0) * (double)st[2] + (double)d;
  if (ext >= 4.6e18) return fail(CP_EINVAL, "%s spans more than 2^62 elements with these strides", what);
  return CP_OK;
}

// Checks common to every attention call.
int check_shape(const cp_shape* s) {
  if (!s) return fail(CP_EINVAL, "shape descriptor is null");
  if (s->b < 1 || s->hq < 1 || s->hkv < 1)
    return fail(CP_EINVAL, "b, hq and hkv must be >= 1 (got %d, %d, %d)", s->b, s->hq, s->hkv);
  if (s->hq % s->hkv != 0) return fail(CP_EINVAL, "hq (%d) is not a multiple of hkv (%d)", s->hq, s->hkv);
  if (s->d != 64 && s->d != 128) return fail(CP_EINVAL, "head dimension %d is not 64 or 128", s->d);
  if (s->sq < 0 || s->sk < 0 || s->sq > (INT32_MAX / 2) || s->sk > (INT32_MAX / 2))
    return fail(CP_EINVAL, "row counts sq=%lld sk=%lld outside [0, 2^30)", (long long)s->sq,
                (long long)s->sk);
  // Element counts of q and k/v (and the products the calls form from them)
  // stay below 2^62.
  if ((double)s->b * s->hq * (double)s->sq * s->d >= 4.6e18 || (double)s->b * s->hkv * (double)s->sk * s->d >= 4.6e18)
    return fail(CP_EINVAL, "b x heads x rows x d beyond 2^62 elements");
  if (!std::isfinite(s->scale) || !(s->scale > 0.0f))
    return fail(CP_EINVAL, "scale must be finite and > 0 (got %g)", (double)s->scale);
  if (int rc = check_dtype(s->in_dtype, "in_dtype")) return rc;
  if (int rc = check_dtype(s->out_dtype, "out_dtype")) return rc;
  if (int rc = check_strides(s->q_str, s->in_dtype, "q")) return rc;
  if (int rc = check_strides(s->k_str, s->in_dtype, "k")) return rc;
  if (int rc = check_strides(s->v_str, s->in_dtype, "v")) return rc;
  if (int rc = check_extent(s->b, s->hq, s->sq, s->d, s->q_str, "q")) return rc;
  if (int rc = check_extent(s->b, s->hkv, s->sk, s->d, s->k_str, "k")) return rc;
  if (int rc = check_extent(s->b, s->hkv, s->sk, s->d, s->v_str, "v")) return rc;
  if (int rc = check_extent(s->b, s->hq, s->sq, s->d, s->o_str, "o")) return rc;
  return CP_OK;
}

int check_ptrs16(std::initializer_list<std::pair<const void*, const char*>> ps) {
  for (auto& p : ps) {
    if (!p.first) return fail(CP_EINVAL, "%s is null", p.second);
    if (!aligned16(p.first)) return fail(CP_EINVAL, "%s is not 16-byte aligned", p.second);
  }
  return CP_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return CP_OK;
  return fail(CP_EHIP, "%s: %s", what, hipGetErrorString(e));
}

FwdArgs base_args(const cp_shape* s) {
  FwdArgs a{};
  for (int i = 0; i < 3; ++i) {
    a.q_str[i] = s->q_str[i];
    a.k_str[i] = s->k_str[i];
    a.v_str[i] = s->v_str[i];
    a.o_str[i] = s->o_str[i];
  }
  a.b = s->b;
  a.hq = s->hq;
  a.hkv = s->hkv;
  a.d = s->d;
  a.sq = (int32_t)s->sq;
  a.sk = (int32_t)s->sk;
  a.scale_log2 = (float)((double)s->scale * 1.4426950408889634);
  a.in_dtype = s->in_dtype;
  return a;
}

}  // namespace

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

FwdWorkspace fwd_workspace_layout(int32_t b, int32_t hkv, int32_t d, int64_t sq, int64_t sk, int32_t cp,
                                  int32_t in_dtype) {
  FwdWorkspace w{};
  const int tk = tile_keys(in_dtype);
  const int64_t per = cp > 0 ? sk / cp : 0;
  const int64_t tpr = (per + tk - 1) / tk;
  const int64_t ntiles = tpr * cp;
  w.bounds_off = 0;
  size_t off = align_up((size_t)ntiles * 16, 256);
  w.kpos_off = off;
  if (in_dtype == CP_BF16) off += align_up((size_t)ntiles * tk * 4, 256);
  w.order_off = off;
  if (in_dtype == CP_BF16) off += align_up((size_t)2 * ((sq + kOrderRows - 1) / kOrderRows) * 4, 256);
  w.list_off = off;
  if (fwd_pre_lists(in_dtype, sq, sk, cp)) off += align_up((size_t)((sq + kOrderRows - 1) / kOrderRows) * ntiles * 4, 256);
  w.vt_off = off;
  w.vt_row = ntiles * tk;
  if (fwd_wide_keys(in_dtype, sk)) off += align_up((size_t)b * hkv * d * (size_t)w.vt_row * 2, 256);
  w.total = off < 256 ? 256 : off;
  return w;
}

BwdWorkspace bwd_workspace_layout(int32_t b, int32_t hq, int32_t hkv, int32_t d, int64_t sq, int64_t sk,
                                  int32_t cp) {
  BwdWorkspace w{};
  const int64_t per = cp > 0 ? sk / cp : 0;
  const int64_t tpr = (per + kBwdTile - 1) / kBwdTile;
  const int64_t nkt = tpr * cp;
  w.kt_row = nkt * kBwdTile;
  w.sq_pad = (sq + kBwdTile - 1) / kBwdTile * kBwdTile;
  const int64_t nqt = w.sq_pad / kBwdTile;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes, 256);
    return at;
  };
  w.kbounds_off = take((size_t)nkt * 16);
  w.kpos_off = take((size_t)w.kt_row * 4);
  w.qbounds_off = take((size_t)nqt * 16);
  w.qholes_off = take((size_t)nqt * 8);
  w.qlo_off = take((size_t)w.sq_pad * 4);
  w.qspan_off = take((size_t)w.sq_pad * 4);
  w.nl2_off = take((size_t)b * hq * (size_t)w.sq_pad * 4);
  w.dlt_off = take((size_t)b * hq * (size_t)w.sq_pad * 4);
  w.kvcost_off = off;
  if (bwd_kv_order(sk, cp)) take((size_t)2 * bwd_kv_groups(sk, cp) * 4);
  w.qcost_off = off;
  if (bwd_q_order(sq)) take((size_t)2 * ((sq + 255) / 256) * 4);
  w.total = off < 256 ? 256 : off;
  return w;
}

}  // namespace cpattn

using namespace cpattn;

extern "C" const char* cp_last_error(void) { return g_last_error.c_str(); }

extern "C" int cp_version(void) { return 200; }

extern "C" size_t cp_attn_ring_fwd_workspace(const cp_shape* s, int32_t cp) {
  if (check_shape(s) != CP_OK || cp < 1) return 0;
  return fwd_workspace_layout(s->b, s->hkv, s->d, s->sq, s->sk, cp, s->in_dtype).total;
}

namespace {

// Validates one forward launch and fills its kernel arguments; launches nothing.
int prep_fwd(const cp_shape* s, int32_t cp, int32_t rank, const void* q, const void* k, const void* v,
             const int32_t* q_pos, const int32_t* q_lo, const int32_t* k_pos, void* o, int32_t o_dtype,
             float* lse, void* ws, size_t ws_bytes, FwdArgs* out, bool v_in_place = false) {
  if (int rc = check_ptrs16({{q, "q"}, {o, "o"}, {lse, "lse"}})) return rc;
  if (!q_pos) return fail(CP_EINVAL, "q_pos is null");
  if (s->sk > 0) {
    if (int rc = check_ptrs16({{k, "k"}, {v, "v"}})) return rc;
    if (!k_pos) return fail(CP_EINVAL, "k_pos is null");
  }
  if (int rc = check_strides(s->o_str, o_dtype, "o")) return rc;
  if (s->o_str[2] < s->d) return fail(CP_EINVAL, "o row stride %lld is smaller than d", (long long)s->o_str[2]);
  if (s->sk > 0 && (s->k_str[2] < s->d || s->v_str[2] < s->d))
    return fail(CP_EINVAL, "k/v row strides must be at least d");
  // The bf16 kernel addresses one (batch, kv head) of K and of V with 32-bit
  // buffer offsets.
  if (s->in_dtype == CP_BF16 &&
      ((double)s->sk * (double)s->k_str[2] * 2.0 >= 4294967040.0 ||
       (double)s->sk * (double)s->v_str[2] * 2.0 >= 4294967040.0))
    return fail(CP_EINVAL, "key rows x row stride exceed the 4 GiB reach of one buffer descriptor");
  // Listed key tiles carry the ring rank in 8 bits and the tile index within
  // the rank's shard in 16 bits.
  if (cp > 255) return fail(CP_EINVAL, "cp must be <= 255 (got %d)", cp);
  if ((s->sk / cp + tile_keys(s->in_dtype) - 1) / tile_keys(s->in_dtype) > 65535)
    return fail(CP_EINVAL, "a shard of %lld key rows has more than 65535 key tiles", (long long)(s->sk / cp));
  const FwdWorkspace w = fwd_workspace_layout(s->b, s->hkv, s->d, s->sq, s->sk, cp, s->in_dtype);
  // So does the wide launch's V^T copy: d rows over every key slot of the padded tiles.
  if (!v_in_place && fwd_wide_keys(s->in_dtype, s->sk) && (double)s->d * (double)w.vt_row * 2.0 >= 4294967040.0)
    return fail(CP_EINVAL, "%lld key rows exceed the 4 GiB reach of one buffer descriptor for V^T", (long long)s->sk);
  // Reading V in place, the launch uses the tables only (the workspace up to its V^T part).
  // Reading V in place needs only the tables; the key lists are then used
  // when they fit as well.
  const size_t need = v_in_place ? w.list_off : w.total;
  if (!ws) return fail(CP_EWORKSPACE, "workspace is null (%zu bytes needed)", need);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(CP_EWORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < need) return fail(CP_EWORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  FwdArgs a = base_args(s);
  a.q = q;
  a.k = k;
  a.v = v;
  a.q_pos = q_pos;
  a.q_lo = q_lo;
  a.k_pos = k_pos;
  a.o = o;
  a.lse = lse;
  a.cp = cp;
  a.rank = rank;
  a.rows_per_rank = (int32_t)(s->sk / cp);
  const int tk = tile_keys(s->in_dtype);
  a.tiles_per_rank = (a.rows_per_rank + tk - 1) / tk;
  a.out_dtype = o_dtype;
  a.ws = ws;
  a.v_in_place = v_in_place ? 1 : 0;
  a.pre_lists = fwd_pre_lists(s->in_dtype, s->sq, s->sk, cp) && ws_bytes >= w.vt_off ? 1 : 0;
  *out = a;
  return CP_OK;
}

int run_fwd(const cp_shape* s, int32_t cp, int32_t rank, const void* q, const void* k, const void* v,
            const int32_t* q_pos, const int32_t* q_lo, const int32_t* k_pos, void* o, int32_t o_dtype,
            float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (s->sq == 0) return CP_OK;  // no query rows: nothing to read or write
  FwdArgs a;
  if (int rc = prep_fwd(s, cp, rank, q, k, v, q_pos, q_lo, k_pos, o, o_dtype, lse, ws, ws_bytes, &a)) return rc;
  return hip_status(launch_fwd(a, stream), "forward launch");
}

}  // namespace

extern "C" int cp_attn_partial_fwd(const cp_shape* s, const void* q, const void* k, const void* v,
                                   const int32_t* q_pos, const int32_t* q_lo, const int32_t* k_pos, float* o,
                                   float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (int rc = check_shape(s)) return rc;
  return run_fwd(s, 1, 0, q, k, v, q_pos, q_lo, k_pos, o, CP_F32, lse, ws, ws_bytes, stream);
}

extern "C" int cp_attn_ring_fwd(const cp_shape* s, int32_t cp, int32_t rank, const void* q_loc,
                                const void* k_all, const void* v_all, const int32_t* q_pos,
                                const int32_t* q_lo, const int32_t* k_pos_all, void* o, float* lse,
                                void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (int rc = check_shape(s)) return rc;
  if (cp < 1) return fail(CP_EINVAL, "cp must be >= 1 (got %d)", cp);
  if (rank < 0 || rank >= cp) return fail(CP_EINVAL, "rank %d outside [0, %d)", rank, cp);
  if (s->sk % (2 * (int64_t)cp) != 0)
    return fail(CP_ESHAPE, "key rows %lld are not a multiple of 2*cp = %lld", (long long)s->sk,
                2 * (long long)cp);
  return run_fwd(s, cp, rank, q_loc, k_all, v_all, q_pos, q_lo, k_pos_all, o, s->out_dtype, lse, ws,
                 ws_bytes, stream);
}

extern "C" int cp_attn_ring_fwd_noalloc(const cp_shape* s, int32_t cp, int32_t rank, const void* q_loc,
                                        const void* k_all, const void* v_all, const int32_t* q_pos,
                                        const int32_t* q_lo, const int32_t* k_pos_all, void* o, float* lse,
                                        hipStream_t stream) {
  clear_error();
  if (int rc = check_shape(s)) return rc;
  if (cp < 1) return fail(CP_EINVAL, "cp must be >= 1 (got %d)", cp);
  if (rank < 0 || rank >= cp) return fail(CP_EINVAL, "rank %d outside [0, %d)", rank, cp);
  if (s->sk % (2 * (int64_t)cp) != 0)
    return fail(CP_ESHAPE, "key rows %lld are not a multiple of 2*cp = %lld", (long long)s->sk,
                2 * (long long)cp);
  if (s->sq == 0) return CP_OK;
  // The tables of the launch that reads V in place: the workspace without its
  // V^T part and without the per-query-tile key lists (used when they fit).
  const FwdWorkspace w = fwd_workspace_layout(s->b, s->hkv, s->d, s->sq, s->sk, cp, s->in_dtype);
  const size_t need = w.list_off;
  if (need > kNoAllocScratchBytes)
    return fail(CP_EINVAL, "%lld key rows need %zu bytes of tile tables, beyond the %zu-byte static scratch of the "
                "allocation-free forward", (long long)s->sk, need, kNoAllocScratchBytes);
  void* scratch = nullptr;
  if (int rc = hip_status(fwd_noalloc_scratch(&scratch), "static scratch address")) return rc;
  FwdArgs a;
  if (int rc = prep_fwd(s, cp, rank, q_loc, k_all, v_all, q_pos, q_lo, k_pos_all, o, s->out_dtype, lse, scratch,
                        kNoAllocScratchBytes, &a, /*v_in_place=*/true))
    return rc;
  return hip_status(launch_fwd(a, stream), "forward launch");
}

extern "C" int cp_attn_merge(int64_t rows, int32_t d, float* o_acc, float* lse_acc, const float* o_p,
                             const float* lse_p, hipStream_t stream) {
  clear_error();
  if (rows < 0) return fail(CP_EINVAL, "rows must be >= 0 (got %lld)", (long long)rows);
  if (rows > (int64_t)1 << 31) return fail(CP_EINVAL, "rows %lld exceed 2^31", (long long)rows);
  if (d != 64 && d != 128) return fail(CP_EINVAL, "head dimension %d is not 64 or 128", d);
  if (int rc = check_ptrs16({{o_acc, "o_acc"}, {o_p, "o_p"}})) return rc;
  if (!lse_acc || !lse_p) return fail(CP_EINVAL, "lse pointer is null");
  if (rows == 0) return CP_OK;
  return hip_status(launch_merge(rows, d, o_acc, lse_acc, o_p, lse_p, stream), "merge launch");
}

namespace {

// Workspace of the stepwise ring: the step's partial O and LSE, then the
// tables of the step kernel (cp = 1 over one shard).
struct StepwiseLayout {
  size_t kern_off, kern_bytes, total;
};

StepwiseLayout stepwise_layout(const cp_shape* s, int32_t cp) {
  StepwiseLayout w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes, 256);
    return at;
  };
  w.kern_bytes = fwd_workspace_layout(s->b, s->hkv, s->d, s->sq, s->sk / cp, 1, s->in_dtype).total;
  w.kern_off = take(w.kern_bytes);
  w.total = off;
  return w;
}

// One staged shard of K or V: [b][hkv][sk/cp][d] packed, 256-byte aligned.
size_t stage_slot_bytes(const cp_shape* s, int32_t cp) {
  return align_up((size_t)s->b * s->hkv * (size_t)(s->sk / cp) * s->d * esize(s->in_dtype), 256);
}

// Copies rows [src*R, (src+1)*R) of every (batch, kv head) of x (element
// strides st, rows contiguous) into dst, packed as [b][hkv][R][d].
hipError_t copy_shard(char* dst, const void* x, const int64_t* st, const cp_shape* s, int64_t R, int32_t src,
                      hipStream_t stream) {
  const size_t e = esize(s->in_dtype);
  const size_t width = (size_t)R * s->d * e;
  if (width == 0) return hipSuccess;
  for (int32_t b = 0; b < s->b; ++b) {
    const char* from = static_cast<const char*>(x) + ((size_t)b * st[0] + (size_t)src * R * st[2]) * e;
    char* to = dst + (size_t)b * s->hkv * width;
    const hipError_t err =
        hipMemcpy2DAsync(to, width, from, (size_t)st[1] * e, width, s->hkv, hipMemcpyDeviceToDevice, stream);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

// Events of one call, released when the call returns (a recorded event that
// has not completed yet is released by the runtime once it completes).
struct CallEvents {
  std::vector<hipEvent_t> ev;
  hipError_t make(hipEvent_t* out) {
    const hipError_t e = hipEventCreateWithFlags(out, hipEventDisableTiming);
    if (e == hipSuccess) ev.push_back(*out);
    return e;
  }
  ~CallEvents() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  }
};

}  // namespace

extern "C" size_t cp_attn_ring_fwd_stepwise_workspace(const cp_shape* s, int32_t cp) {
  if (check_shape(s) != CP_OK || cp < 1) return 0;
  return stepwise_layout(s, cp).total;
}

extern "C" size_t cp_attn_ring_stage_bytes(const cp_shape* s, int32_t cp) {
  if (check_shape(s) != CP_OK || cp < 1) return 0;
  const size_t n = 4 * stage_slot_bytes(s, cp);  // two slots of K and V
  return n < 256 ? 256 : n;
}

extern "C" int cp_attn_ring_fwd_stepwise(const cp_shape* s, int32_t cp, int32_t rank, const void* q_loc,
                                         const void* k_all, const void* v_all, const int32_t* q_pos,
                                         const int32_t* q_lo, const int32_t* k_pos_all, float* o, float* lse,
                                         void* ws, size_t ws_bytes, void* stage, size_t stage_bytes,
                                         hipStream_t stream, hipStream_t copy_stream) {
  clear_error();
  if (int rc = check_shape(s)) return rc;
  if (cp < 1) return fail(CP_EINVAL, "cp must be >= 1 (got %d)", cp);
  if (rank < 0 || rank >= cp) return fail(CP_EINVAL, "rank %d outside [0, %d)", rank, cp);
  if (s->sk % (2 * (int64_t)cp) != 0)
    return fail(CP_ESHAPE, "key rows %lld are not a multiple of 2*cp = %lld", (long long)s->sk,
                2 * (long long)cp);
  if (s->out_dtype != CP_F32) return fail(CP_EDTYPE, "the stepwise ring writes an fp32 O (out_dtype must be CP_F32)");
  if (s->o_str[2] != s->d || s->o_str[1] != s->sq * s->d || s->o_str[0] != s->hq * s->sq * s->d)
    return fail(CP_EINVAL, "o must be contiguous [b, hq, sq, d] for the merge");
  if (s->sq == 0) return CP_OK;
  const int64_t R = s->sk / cp;
  const StepwiseLayout w = stepwise_layout(s, cp);
  if (!ws) return fail(CP_EWORKSPACE, "workspace is null (%zu bytes needed)", w.total);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(CP_EWORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < w.total) return fail(CP_EWORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, w.total);
  const size_t slot = stage_slot_bytes(s, cp);
  if (stage) {
    if ((reinterpret_cast<uintptr_t>(stage) & 255u) != 0)
      return fail(CP_EWORKSPACE, "stage is not 256-byte aligned");
    if (stage_bytes < 4 * slot) return fail(CP_EWORKSPACE, "stage too small: %zu < %zu bytes", stage_bytes, 4 * slot);
    if (s->k_str[2] != s->d || s->v_str[2] != s->d || s->k_str[1] < s->sk * s->d || s->v_str[1] < s->sk * s->d)
      return fail(CP_EINVAL, "staging copies need k_all and v_all with contiguous rows and heads of sk rows");
  }
  char* wsb = static_cast<char*>(ws);
  void* kws = wsb + w.kern_off;
  const size_t e = esize(s->in_dtype);
  char* st = static_cast<char*>(stage);

  // Every step's launch is validated before anything is enqueued.
  std::vector<FwdArgs> steps(cp);
  for (int32_t t = 0; t < cp; ++t) {
    int32_t src = rank - t;
    if (src < 0) src += cp;
    cp_shape ss = *s;
    ss.sk = R;
    const void* k = static_cast<const char*>(k_all) + (size_t)src * R * s->k_str[2] * e;
    const void* v = static_cast<const char*>(v_all) + (size_t)src * R * s->v_str[2] * e;
    if (stage && t > 0) {
      char* kb = st + (size_t)(t & 1) * 2 * slot;
      k = kb;
      v = kb + slot;
      const int64_t packed[3] = {(int64_t)s->hkv * R * s->d, R * s->d, s->d};
      for (int i = 0; i < 3; ++i) ss.k_str[i] = ss.v_str[i] = packed[i];
    }
    // Step 0 writes (o, lse); every later step merges its partial into them
    // in the kernel's epilogue.
    if (int rc = prep_fwd(&ss, 1, 0, q_loc, k, v, q_pos, q_lo, k_pos_all + (size_t)src * R, o, CP_F32, lse, kws,
                          w.kern_bytes, &steps[t]))
      return rc;
    steps[t].merge_acc = t > 0 ? 1 : 0;
  }

  const bool staged = stage != nullptr && cp > 1;
  CallEvents ev;
  std::vector<hipEvent_t> copied(cp, nullptr);
  hipEvent_t slot_free[2] = {nullptr, nullptr}, start = nullptr, joined = nullptr;
  if (staged) {
    if (int rc = hip_status(ev.make(&start), "event")) return rc;
    if (int rc = hip_status(ev.make(&joined), "event")) return rc;
    for (int i = 0; i < 2; ++i)
      if (int rc = hip_status(ev.make(&slot_free[i]), "event")) return rc;
    for (int32_t t = 1; t < cp; ++t)
      if (int rc = hip_status(ev.make(&copied[t]), "event")) return rc;
    // The shards are read only after the work already queued on stream.
    if (int rc = hip_status(hipEventRecord(start, stream), "event record")) return rc;
    if (int rc = hip_status(hipStreamWaitEvent(copy_stream, start, 0), "stream wait")) return rc;
  }
  // Copy of step t's shard into slot t % 2, after step t - 2 (the slot's last
  // reader) has finished.
  auto enqueue_copy = [&](int32_t t) -> int {
    int32_t src = rank - t;
    if (src < 0) src += cp;
    char* kb = st + (size_t)(t & 1) * 2 * slot;
    if (t >= 3)
      if (int rc = hip_status(hipStreamWaitEvent(copy_stream, slot_free[t & 1], 0), "stream wait")) return rc;
    if (int rc = hip_status(copy_shard(kb, k_all, s->k_str, s, R, src, copy_stream), "K copy")) return rc;
    if (int rc = hip_status(copy_shard(kb + slot, v_all, s->v_str, s, R, src, copy_stream), "V copy")) return rc;
    return hip_status(hipEventRecord(copied[t], copy_stream), "event record");
  };
  if (staged)
    if (int rc = enqueue_copy(1)) return rc;
  for (int32_t t = 0; t < cp; ++t) {
    if (staged && t + 1 < cp && t + 1 >= 2)
      if (int rc = enqueue_copy(t + 1)) return rc;
    if (staged && t > 0)
      if (int rc = hip_status(hipStreamWaitEvent(stream, copied[t], 0), "stream wait")) return rc;
    if (int rc = hip_status(launch_fwd(steps[t], stream), "forward launch")) return rc;
    if (staged && t > 0)
      if (int rc = hip_status(hipEventRecord(slot_free[t & 1], stream), "event record")) return rc;
  }
  if (staged) {
    if (int rc = hip_status(hipEventRecord(joined, copy_stream), "event record")) return rc;
    if (int rc = hip_status(hipStreamWaitEvent(stream, joined, 0), "stream wait")) return rc;
  }
  return CP_OK;
}

namespace {

int check_a2a(int32_t g, int32_t heads, int64_t rows, int32_t d, int32_t dtype) {
  if (g < 1) return fail(CP_EINVAL, "group size g must be >= 1 (got %d)", g);
  if (heads < 1 || heads > 65535) return fail(CP_EINVAL, "heads must be in [1, 65535] (got %d)", heads);
  if (heads % g != 0) return fail(CP_EINVAL, "heads %d is not a multiple of g = %d", heads, g);
  if (rows < 0) return fail(CP_EINVAL, "rows must be >= 0 (got %lld)", (long long)rows);
  if (rows > (int64_t)1 << 31) return fail(CP_EINVAL, "rows %lld exceed 2^31", (long long)rows);
  if (d != 64 && d != 128) return fail(CP_EINVAL, "head dimension %d is not 64 or 128", d);
  return check_dtype(dtype, "dtype");
}

}  // namespace

extern "C" int cp_a2a_pack(int32_t g, int32_t heads, int64_t rows, int32_t d, int32_t dtype, void* x,
                           int64_t x_row_stride, void* send, int32_t inverse, hipStream_t stream) {
  clear_error();
  if (int rc = check_a2a(g, heads, rows, d, dtype)) return rc;
  if (x_row_stride < (int64_t)heads * d)
    return fail(CP_EINVAL, "x row stride %lld is smaller than heads*d = %lld", (long long)x_row_stride,
                (long long)heads * d);
  if (x_row_stride % (16 / (int64_t)esize(dtype)) != 0)
    return fail(CP_EINVAL, "x row stride is not a multiple of 16 bytes");
  if ((double)rows * (double)x_row_stride * esize(dtype) >= 4.6e18)
    return fail(CP_EINVAL, "x spans more than 2^62 bytes with this row stride");
  if (rows == 0) return CP_OK;
  if (int rc = check_ptrs16({{x, "x"}, {send, "send"}})) return rc;
  return hip_status(inverse ? launch_a2a(g, heads, rows, d, dtype, send, x, x_row_stride, 0, 0, stream)
                            : launch_a2a(g, heads, rows, d, dtype, x, send, x_row_stride, 0, 1, stream),
                    "a2a pack launch");
}

extern "C" int cp_a2a_unpack(int32_t g, int32_t heads, int64_t rows, int32_t d, int32_t dtype, void* recv,
                             void* y, int32_t inverse, hipStream_t stream) {
  clear_error();
  if (int rc = check_a2a(g, heads, rows, d, dtype)) return rc;
  if (rows == 0) return CP_OK;
  if (int rc = check_ptrs16({{recv, "recv"}, {y, "y"}})) return rc;
  return hip_status(inverse ? launch_a2a(g, heads, rows, d, dtype, y, recv, 0, 1, 1, stream)
                            : launch_a2a(g, heads, rows, d, dtype, recv, y, 0, 1, 0, stream),
                    "a2a unpack launch");
}

extern "C" size_t cp_attn_bwd_workspace(const cp_shape* s, int32_t cp) {
  if (check_shape(s) != CP_OK || cp < 1) return 0;
  return bwd_workspace_layout(s->b, s->hq, s->hkv, s->d, s->sq, s->sk, cp).total;
}

extern "C" int cp_attn_bwd_delta(const cp_shape* s, const void* dout, const void* o, float* delta,
                                 hipStream_t stream) {
  clear_error();
  if (int rc = check_shape(s)) return rc;
  if (s->in_dtype != CP_BF16) return fail(CP_EDTYPE, "the backward takes bf16 inputs (in_dtype must be CP_BF16)");
  if (s->sq == 0) return CP_OK;
  if (int rc = check_ptrs16({{dout, "dout"}, {o, "o"}})) return rc;
  if (!delta) return fail(CP_EINVAL, "delta is null");
  if (int rc = check_strides(s->o_str, s->out_dtype, "o")) return rc;
  if (s->o_str[2] < s->d || s->q_str[2] < s->d) return fail(CP_EINVAL, "dout/o row strides must be at least d");
  // The kernel indexes rows in 32 bits; 2^31 rows of bf16 dO and O would
  // already take over 500 GB at d = 64.
  if ((int64_t)s->b * s->hq * s->sq >= (int64_t)1 << 31)
    return fail(CP_EINVAL, "b x hq x sq = %lld rows reach 2^31", (long long)((int64_t)s->b * s->hq * s->sq));
  BwdArgs a{};
  for (int i = 0; i < 3; ++i) {
    a.q_str[i] = s->q_str[i];
    a.o_str[i] = s->o_str[i];
  }
  a.dout = dout;
  a.o = o;
  a.delta_out = delta;
  a.b = s->b;
  a.hq = s->hq;
  a.d = s->d;
  a.sq = (int32_t)s->sq;
  a.out_dtype = s->out_dtype;
  return hip_status(launch_delta(a, stream), "delta launch");
}

namespace {

int run_bwd(const cp_shape* s, int32_t cp, int32_t rank, const void* q, const void* k, const void* v,
            const void* dout, const float* lse, const float* delta, const int32_t* q_pos, const int32_t* q_lo,
            const int32_t* k_pos, float* dq, float* dk, float* dv, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (s->in_dtype != CP_BF16) return fail(CP_EDTYPE, "the backward takes bf16 inputs (in_dtype must be CP_BF16)");
  if (cp > 255) return fail(CP_EINVAL, "cp must be <= 255 (got %d)", cp);
  if (s->sq == 0 || s->sk == 0) return CP_OK;  // no allowed pair: every gradient contribution is zero
  if (int rc = check_ptrs16({{q, "q"}, {k, "k"}, {v, "v"}, {dout, "dout"}, {dq, "dq"}, {dk, "dk"}, {dv, "dv"}}))
    return rc;
  if (!lse || !delta) return fail(CP_EINVAL, "lse or delta is null");
  if (!q_pos || !k_pos) return fail(CP_EINVAL, "q_pos or k_pos is null");
  if (s->q_str[2] < s->d || s->k_str[2] < s->d || s->v_str[2] < s->d)
    return fail(CP_EINVAL, "q/k/v row strides must be at least d");
  const int64_t per = s->sk / cp;
  if ((per + kBwdTile - 1) / kBwdTile > 65535)
    return fail(CP_EINVAL, "a shard of %lld key rows has more than 65535 key tiles", (long long)per);
  // The dK/dV kernel lists (query head, query tile) pairs in 16 + 15 bits.
  if ((s->sq + kBwdTile - 1) / kBwdTile > 65535 || s->hq / s->hkv > 32767)
    return fail(CP_EINVAL, "%lld query rows or %d query heads per kv head are too many for the backward",
                (long long)s->sq, s->hq / s->hkv);
  const BwdWorkspace w = bwd_workspace_layout(s->b, s->hq, s->hkv, s->d, s->sq, s->sk, cp);
  // The kernels address the padded per-row and per-key arrays, one tile's
  // rows of Q, dO, K or V, and the dK/dV workgroup's 256 rows of V, with
  // 32-bit buffer offsets.
  if ((double)w.kt_row * 4.0 >= 2147483648.0 || (double)s->b * s->hq * (double)w.sq_pad * 4.0 >= 2147483648.0 ||
      64.0 * (double)s->q_str[2] * 2.0 >= 2147483648.0 || 64.0 * (double)s->k_str[2] * 2.0 >= 2147483648.0 ||
      256.0 * (double)s->v_str[2] * 2.0 >= 2147483648.0)
    return fail(CP_EINVAL, "sequence too long for 32-bit buffer offsets (sq=%lld, sk=%lld)", (long long)s->sq,
                (long long)s->sk);
  if (!ws) return fail(CP_EWORKSPACE, "workspace is null (%zu bytes needed)", w.total);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(CP_EWORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < w.total) return fail(CP_EWORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, w.total);
  BwdArgs a{};
  for (int i = 0; i < 3; ++i) {
    a.q_str[i] = s->q_str[i];
    a.k_str[i] = s->k_str[i];
    a.v_str[i] = s->v_str[i];
  }
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.q_pos = q_pos;
  a.q_lo = q_lo;
  a.k_pos = k_pos;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.b = s->b;
  a.hq = s->hq;
  a.hkv = s->hkv;
  a.d = s->d;
  a.sq = (int32_t)s->sq;
  a.sk = (int32_t)s->sk;
  a.cp = cp;
  a.rank = rank;
  a.rows_per_rank = (int32_t)per;
  a.scale = s->scale;
  a.ws = ws;
  return hip_status(launch_bwd(a, stream), "backward launch");
}

}  // namespace

extern "C" int cp_attn_partial_bwd(const cp_shape* s, const void* q, const void* k, const void* v, const void* dout,
                                   const float* lse, const float* delta, const int32_t* q_pos, const int32_t* q_lo,
                                   const int32_t* k_pos, float* dq, float* dk, float* dv, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  clear_error();
  if (int rc = check_shape(s)) return rc;
  return run_bwd(s, 1, 0, q, k, v, dout, lse, delta, q_pos, q_lo, k_pos, dq, dk, dv, ws, ws_bytes, stream);
}

extern "C" int cp_attn_ring_bwd(const cp_shape* s, int32_t cp, int32_t rank, const void* q_loc, const void* k_all,
                                const void* v_all, const void* dout, const float* lse, const float* delta,
                                const int32_t* q_pos, const int32_t* q_lo, const int32_t* k_pos_all, float* dq,
                                float* dk_all, float* dv_all, void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (int rc = check_shape(s)) return rc;
  if (cp < 1) return fail(CP_EINVAL, "cp must be >= 1 (got %d)", cp);
  if (rank < 0 || rank >= cp) return fail(CP_EINVAL, "rank %d outside [0, %d)", rank, cp);
  if (s->sk % (2 * (int64_t)cp) != 0)
    return fail(CP_ESHAPE, "key rows %lld are not a multiple of 2*cp = %lld", (long long)s->sk, 2 * (long long)cp);
  return run_bwd(s, cp, rank, q_loc, k_all, v_all, dout, lse, delta, q_pos, q_lo, k_pos_all, dq, dk_all, dv_all, ws,
                 ws_bytes, stream);
}
