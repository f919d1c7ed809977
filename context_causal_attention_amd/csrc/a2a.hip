// Head exchange of the all-to-all level of hierarchical context parallelism
// (NeMo Megatron-Bridge "Hierarchical Context Parallel Skill": with
// cp_comm_type "a2a+p2p" the first level is a group of g ranks that
// communicate all-to-all).  Before the exchange a rank holds every head of its
// rows; after it, every row of the group for H/g of the heads.  These kernels
// are the rank-local halves: packing the sequence shard into the per-rank send
// blocks, and unpacking the received blocks into the [heads, rows, d] layout
// the attention calls read (and the inverse of each).
//
// Pure data movement, bound by HBM bandwidth: each row of d elements (128 to
// 512 bytes) is moved whole as 16-byte vectors, with ordinary loads and stores
// (nontemporal hints measured 10-25% slower here).  Grid y is the head-block row
// (packed layout [g][H/g] = [H] rows of `rows` rows each), grid x covers the
// rows in a grid-stride loop, so every lane's addresses come from one division
// by a compile-time constant.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "internal.h"

namespace cpattn {
namespace a2ak {

using dev::u32x4;

struct RowMap {
  const char* src;
  char* dst;
  int64_t rows;        // rows per head block
  int64_t row_bytes;   // d * element size
  int64_t x_rs_bytes;  // pack: row stride of the sequence shard, bytes
  int32_t g, hg;       // group size, heads per rank
  int32_t unpack;      // 0: pack ([rows, H, d] side), 1: unpack ([H/g, g*rows, d] side)
  int32_t to_packed;   // 1: the packed [g][H/g][rows][d] layout is the destination
};

// VPR 16-byte vectors per row.
template <int VPR>
__global__ __launch_bounds__(256) void rows_kernel(RowMap m) {
  const int hd = blockIdx.y;  // head index in [g][H/g] order
  const int64_t n = m.rows * VPR;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < n; v += stride) {
    const int64_t t = v / VPR;
    const int c = (int)(v - t * VPR);
    const int64_t packed = ((int64_t)hd * m.rows + t) * m.row_bytes + 16 * c;
    int64_t other;
    if (!m.unpack) {
      other = t * m.x_rs_bytes + (int64_t)hd * m.row_bytes + 16 * c;  // x[t, hd]
    } else {
      const int i = hd / m.hg, hh = hd - i * m.hg;  // block i of head hh
      other = ((int64_t)hh * m.g * m.rows + (int64_t)i * m.rows + t) * m.row_bytes + 16 * c;  // y[hh, i*rows + t]
    }
    const int64_t so = m.to_packed ? other : packed;
    const int64_t dof = m.to_packed ? packed : other;
    const u32x4 val = *reinterpret_cast<const u32x4*>(m.src + so);
    *reinterpret_cast<u32x4*>(m.dst + dof) = val;
  }
}

}  // namespace a2ak

hipError_t launch_a2a(int32_t g, int32_t heads, int64_t rows, int32_t d, int32_t dtype, const void* src, void* dst,
                      int64_t x_row_stride, int32_t unpack, int32_t to_packed, hipStream_t stream) {
  a2ak::RowMap m;
  const int e = dtype == CP_BF16 ? 2 : 4;
  m.src = static_cast<const char*>(src);
  m.dst = static_cast<char*>(dst);
  m.rows = rows;
  m.row_bytes = (int64_t)d * e;
  m.x_rs_bytes = x_row_stride * e;
  m.g = g;
  m.hg = heads / g;
  m.unpack = unpack;
  m.to_packed = to_packed;
  const int vpr = (int)(m.row_bytes / 16);
  // Grid x covers up to 2^22 workgroups (2^30 vectors, the whole row range of
  // every shard up to 2^25 rows at 512 bytes a row); larger shards loop, so the
  // grid's work-item count stays inside its 32-bit limit for every row count.
  const dim3 grid(stride_blocks(rows * vpr), (unsigned)heads);
  switch (vpr) {
    case 8: a2ak::rows_kernel<8><<<grid, 256, 0, stream>>>(m); break;
    case 16: a2ak::rows_kernel<16><<<grid, 256, 0, stream>>>(m); break;
    case 32: a2ak::rows_kernel<32><<<grid, 256, 0, stream>>>(m); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace cpattn
