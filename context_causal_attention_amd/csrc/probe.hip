// Throughput probes of the gfx950 units the attention kernels lean on, for the
// measurement harness only (libcpattn_probe.so; not part of the C ABI of
// libcpattn.so).  Each probe runs one workgroup of 8 wave64s per CU (two waves
// per SIMD, as the attention kernels run) over a fixed number of iterations of
// independent work, so the time measures issue and execution rates, not
// latency:
//   kind 0  MFMA only: v_mfma_f32_32x32x16_bf16 on 4 independent accumulators
//           per wave (32768 flop each);
//   kind 1  exp only: v_exp_f32 on 8 independent chains per lane;
//   kind 2  FMA only: v_fma_f32 on 8 independent chains per lane;
//   kind 3  the forward's inner mix in every wave: per MFMA, 2 FMA, 2 exp,
//           1 bf16 pack and 2 adds (the exponentials of two scores);
//   kind 4  the same work split by wave: waves 0-3 (one per SIMD) issue only
//           the MFMAs, waves 4-7 only the vector part, so a SIMD's matrix
//           work and vector work come from different waves;
//   kind 5  MFMA only, one accumulator chain per wave (each MFMA depends on
//           the previous one);
//   kind 9  as kind 3 with two MFMAs per step (the forward's own ratio: per
//           pair of scores, one score MFMA and one P V MFMA);
//   kinds 6, 7, 8  as 3, 4 and 0 with the MFMA accumulators held in the
//           accumulation registers (AGPRs) instead of VGPRs (the MFMAs are
//           written as inline assembly with an AGPR operand; the results are
//           read only after the loop, behind enough wait states);
//   kinds 10, 11, 12  as 0, 3 and 9 (8 steps an iteration) with each MFMA's
//           A operand read from LDS (one 16-byte read per lane, 1 KB per wave,
//           four steps ahead), as the attention kernels read their K and V
//           tiles;
//   kind 13  as 11 with each exponential replaced by an FMA (same instruction
//           count), to tell the exponential's own cost from the rest of the
//           mix;
//   kind 14  as 11 with the work grouped two steps to a fence (two MFMAs and
//           the vector work of four scores between scheduling barriers).
// Results are written to out so that no work is dropped.  Wave 0 of every
// workgroup also records the shader clock counter (s_memtime) before and after
// the work, so the host can tell the clock the probe ran at: cycles over the
// kernel's duration.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x2 __attribute__((__vector_size__(2 * sizeof(float))));

__device__ __forceinline__ bf16x8 seed_operand(int salt) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (__bf16)(0.001f * (float)((threadIdx.x * 7 + i * 3 + salt) & 15));
  return v;
}

// acc += A B with acc in AGPRs.
__device__ __forceinline__ void mfma_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

__device__ __forceinline__ float fold(const f32x16& a) {
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += a[r];
  return s;
}

template <int KIND>
__global__ __launch_bounds__(512, 1) void probe_kernel(float* out, unsigned long long* clk, int iters) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const bf16x8 a = seed_operand(1), b = seed_operand(2);
  float result = 0.f;
  if constexpr (KIND == 8) {
    f32x16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) mfma_agpr(acc[c], a, b);
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
    for (int c = 0; c < 4; ++c) result += fold(acc[c]);
  } else if constexpr (KIND == 0 || KIND == 5) {
    constexpr int NC = KIND == 0 ? 4 : 1;
    f32x16 acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < NC; ++c) result += fold(acc[c]);
  } else if constexpr (KIND == 1 || KIND == 2) {
    float x[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = 0.01f * (float)(c + (threadIdx.x & 7));
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          // exp2(-x) maps [0, 1] into [0.5, 1]: one v_exp_f32 (negated source) a step
          if constexpr (KIND == 1) x[c] = __builtin_amdgcn_exp2f(-x[c]);
          else x[c] = __builtin_fmaf(x[c], 0.999f, -0.0001f);
        }
#pragma unroll
    for (int c = 0; c < 8; ++c) result += x[c];
  } else {
    // per step: one MFMA and the vector work of two scores (kind 3: both in
    // every wave; kind 4: the MFMAs in waves 0-3, the vector work in 4-7)
    f32x16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
    float s[16], lsum = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s[j] = -0.01f * (float)((threadIdx.x + j) & 31);
    auto ex = [](float x) {
      if constexpr (KIND == 13) return __builtin_fmaf(x, 0.25f, 0.8f);  // in (0.7, 0.9) as exp2 gives
      else return __builtin_amdgcn_exp2f(x);
    };
    auto vec = [&](int m) {
      const float e0 = ex(__builtin_fmaf(s[2 * m], 0.18f, -0.5f));
      const float e1 = ex(__builtin_fmaf(s[2 * m + 1], 0.18f, -0.5f));
      const bf16x2 pk = __builtin_convertvector((f32x2){e0, e1}, bf16x2);
      lsum += e0 + e1;
      // The pair's bf16 bits read as fp32 are about e1 (its high half), so the
      // pack feeds the next step and stays live; 2^(0.18 x - 0.5) keeps every
      // value in (0.7, 0.9).
      s[2 * m] = __builtin_bit_cast(float, pk);
      s[2 * m + 1] = e1;
    };
    constexpr bool AG = KIND >= 6 && KIND <= 8;
    auto mm = [&](int m) {
      if constexpr (AG) mfma_agpr(acc[m & 3], a, b);
      else acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[m & 3], 0, 0, 0);
    };
    if constexpr (KIND >= 10) {
      __shared__ bf16x8 lbuf[2048];
      for (int j = threadIdx.x; j < 2048; j += 512) lbuf[j] = seed_operand(j & 15);
      __syncthreads();
      const int lane = threadIdx.x & 63;
      constexpr int NR = KIND == 12 ? 2 : 1;  // MFMAs (and LDS reads) per step
      constexpr int FENCE = KIND == 14 ? 2 : 1;  // steps between scheduling barriers
      constexpr int PF = 4;                   // steps read ahead
      // read r: 1 KB block r % 32 of the buffer, lane l its 16 bytes l
      auto ld = [&](int r) { return lbuf[((r & 31) << 6) + lane]; };
      bf16x8 op[8][NR];  // step m's operands in op[m % 8]
#pragma unroll
      for (int q = 0; q < PF; ++q)
#pragma unroll
        for (int n = 0; n < NR; ++n) op[q][n] = ld(q * NR + n);
      for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int m = 0; m < 8; ++m) {
#pragma unroll
          for (int n = 0; n < NR; ++n) op[(m + PF) & 7][n] = ld((i * 8 + m + PF) * NR + n);
#pragma unroll
          for (int n = 0; n < NR; ++n)
            acc[(m * NR + n) & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[m & 7][n], b, acc[(m * NR + n) & 3], 0, 0, 0);
          if constexpr (KIND != 10) vec(m);
          if (m % FENCE == FENCE - 1) __builtin_amdgcn_sched_barrier(0);
        }
    } else if (KIND == 3 || KIND == 6) {
      for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          mm(m);
          vec(m);
          __builtin_amdgcn_sched_barrier(0);
        }
    } else if (KIND == 9) {
      for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          mm(m);
          mm(m + 1);
          vec(m);
          __builtin_amdgcn_sched_barrier(0);
        }
    } else if (wave < 4) {
      for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int m = 0; m < 8; ++m) mm(m);
    } else {
      for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int m = 0; m < 8; ++m) vec(m);
    }
    if constexpr (AG) asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
    for (int c = 0; c < 4; ++c) result += fold(acc[c]);
#pragma unroll
    for (int j = 0; j < 16; ++j) result += s[j];
    result += lsum;
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = result;
  if (threadIdx.x == 0) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    clk[2 * blockIdx.x] = t0;
    clk[2 * blockIdx.x + 1] = t1;
  }
}

// The dQ reduction traffic a single-pass backward would make: the dK/dV
// kernel's grid (one workgroup per 256 keys of a kv head, dealt to the XCDs as
// that kernel deals them) walks its query heads and 64-row query tiles in the
// same order, and for every tile holding a query at or after its first key
// (the causal rule of a dense ring) adds a 64 x 128 fp32 block into dQ with
// global float atomics, as the workgroup's reduced partial would be added.
__global__ __launch_bounds__(512, 1) void dq_atomics_kernel(const int* __restrict__ q_pos, const int* __restrict__ k_pos,
                                                            float* __restrict__ dq, int sq, int R, int cp, int hkv,
                                                            int g, float val) {
  constexpr int KPW = 256, QT = 64, D = 128;
  const int tg = (R + KPW - 1) / KPW;
  const int nblk = gridDim.x, bid = blockIdx.x;
  const int per_xcd = nblk / 8;
  int logical = bid < per_xcd * 8 ? (bid % 8) * per_xcd + bid / 8 : bid;
  const int grp = logical % (cp * tg);
  const int kvh = (logical / (cp * tg)) % hkv;
  const int src = grp / tg, ig = grp - src * tg;
  const int key0 = src * R + ig * KPW;
  const int nkeys = min(KPW, R - ig * KPW);
  __shared__ int sMin[8];
  // smallest key position of the workgroup
  int kmin = INT_MAX;
  for (int k = threadIdx.x; k < nkeys; k += 512) kmin = min(kmin, k_pos[key0 + k]);
  for (int o = 1; o < 64; o <<= 1) kmin = min(kmin, __shfl_xor(kmin, o));
  if ((threadIdx.x & 63) == 0) sMin[threadIdx.x >> 6] = kmin;
  __syncthreads();
  kmin = sMin[0];
  for (int w = 1; w < 8; ++w) kmin = min(kmin, sMin[w]);
  const int nqt = (sq + QT - 1) / QT;
  for (int hg = 0; hg < g; ++hg) {
    float* head = dq + (long long)(kvh * g + hg) * sq * D;
    for (int t = 0; t < nqt; ++t) {
      // largest query position of the tile (64 rows, one per lane of wave 0's
      // view; every wave reads them, so no barrier is needed)
      const int r = t * QT + (threadIdx.x & 63);
      int qmax = r < sq ? q_pos[r] : INT_MIN;
      for (int o = 1; o < 64; o <<= 1) qmax = max(qmax, __shfl_xor(qmax, o));
      if (qmax < kmin) continue;
      const int rows = min(QT, sq - t * QT);
      float* blk = head + (long long)t * QT * D;
      for (int e = threadIdx.x; e < rows * D; e += 512) atomicAdd(blk + e, val);
    }
  }
}

}  // namespace

// Runs dq_atomics_kernel over the dK/dV grid of a dense causal ring (cp shards
// of R keys, hkv kv heads of g query heads each, sq query rows of positions
// q_pos, keys of positions k_pos, all device); dq (device) holds hkv * g * sq
// * 128 floats.  Returns a hipError_t.
extern "C" int cp_probe_dq_atomics(const int* q_pos, const int* k_pos, float* dq, int sq, int R, int cp, int hkv,
                                   int g, hipStream_t stream) {
  const int tg = (R + 255) / 256;
  hipLaunchKernelGGL(dq_atomics_kernel, dim3((unsigned)(cp * tg * hkv)), dim3(512), 0, stream, q_pos, k_pos, dq,
                     sq, R, cp, hkv, g, 1.0f / 1024);
  return (int)hipGetLastError();
}

// Runs probe `kind` on `blocks` workgroups of 512 threads with `iters`
// iterations; out (device) holds blocks * 512 floats, clk (device) 2 * blocks
// clock readings (start and end of each workgroup).  Returns a hipError_t.
extern "C" int cp_probe_run(int kind, int blocks, int iters, float* out, unsigned long long* clk,
                            hipStream_t stream) {
  const dim3 g(blocks), t(512);
  switch (kind) {
    case 0: hipLaunchKernelGGL(probe_kernel<0>, g, t, 0, stream, out, clk, iters); break;
    case 1: hipLaunchKernelGGL(probe_kernel<1>, g, t, 0, stream, out, clk, iters); break;
    case 2: hipLaunchKernelGGL(probe_kernel<2>, g, t, 0, stream, out, clk, iters); break;
    case 3: hipLaunchKernelGGL(probe_kernel<3>, g, t, 0, stream, out, clk, iters); break;
    case 4: hipLaunchKernelGGL(probe_kernel<4>, g, t, 0, stream, out, clk, iters); break;
    case 5: hipLaunchKernelGGL(probe_kernel<5>, g, t, 0, stream, out, clk, iters); break;
    case 6: hipLaunchKernelGGL(probe_kernel<6>, g, t, 0, stream, out, clk, iters); break;
    case 7: hipLaunchKernelGGL(probe_kernel<7>, g, t, 0, stream, out, clk, iters); break;
    case 8: hipLaunchKernelGGL(probe_kernel<8>, g, t, 0, stream, out, clk, iters); break;
    case 9: hipLaunchKernelGGL(probe_kernel<9>, g, t, 0, stream, out, clk, iters); break;
    case 10: hipLaunchKernelGGL(probe_kernel<10>, g, t, 0, stream, out, clk, iters); break;
    case 11: hipLaunchKernelGGL(probe_kernel<11>, g, t, 0, stream, out, clk, iters); break;
    case 12: hipLaunchKernelGGL(probe_kernel<12>, g, t, 0, stream, out, clk, iters); break;
    case 13: hipLaunchKernelGGL(probe_kernel<13>, g, t, 0, stream, out, clk, iters); break;
    case 14: hipLaunchKernelGGL(probe_kernel<14>, g, t, 0, stream, out, clk, iters); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}
