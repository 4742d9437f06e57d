// Summary-key pooling: one pyramid level from the level below.
//
// Page 3, paragraph 1 (Le Fil IA / MarkTechPost): keys are cut into contiguous blocks,
// each block is summarised by one summary key obtained from 16 reference queries, and
// the summaries are grouped level by level. Pooling rule (a reading; the page does not
// spell it out): reference query r attends over the node's b children at scale
// tau = 1/sqrt(d), a[r][c] = softmax_c(tau * R[r] . x[c]); the summary is
// sum_c w[c] * x[c] with w[c] = mean_r a[r][c]. Every arithmetic sequence below depends
// only on the node's data, never on where the node sits in a workgroup, so identical
// subtrees give bit-identical summaries.

#include "zha_internal.h"

namespace zha {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kChunk = 64;  // child rows staged in LDS at a time

// z[row][r] = tau * R[r] . x[row] for the `rows` staged rows. Thread -> (row, 4 refs).
template <int D>
__device__ __forceinline__ void pool_scores(const float (*sR)[D], const float (*sX)[D + 4],
                                            float (*sZ)[kNRef + 1], int rows, float tau) {
  const int r = threadIdx.x >> 2;
  const int q0 = (threadIdx.x & 3) * 4;
  if (r < rows) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll 8
    for (int k = 0; k < D; ++k) {
      const float x = sX[r][k];
      a0 = fmaf(sR[q0 + 0][k], x, a0);
      a1 = fmaf(sR[q0 + 1][k], x, a1);
      a2 = fmaf(sR[q0 + 2][k], x, a2);
      a3 = fmaf(sR[q0 + 3][k], x, a3);
    }
    sZ[r][q0 + 0] = tau * a0;
    sZ[r][q0 + 1] = tau * a1;
    sZ[r][q0 + 2] = tau * a2;
    sZ[r][q0 + 3] = tau * a3;
  }
}

template <typename Tin, typename Tr, int D>
__device__ __forceinline__ void stage_R(float (*sR)[D], const Tr* R) {
  for (int i = threadIdx.x; i < kNRef * D; i += kPoolThreads) sR[i / D][i % D] = to_f32(R[i]);
}

template <typename Tin, int D>
__device__ __forceinline__ void stage_rows(float (*sX)[D + 4], const Tin* src, int rows) {
  for (int i = threadIdx.x; i < rows * D; i += kPoolThreads) sX[i / D][i % D] = to_f32(src[i]);
}

// b <= 64: a workgroup pools floor(64 / b) whole nodes from one staged chunk.
template <typename Tin, typename Tr, int D>
__global__ __launch_bounds__(kPoolThreads) void pool_small_kernel(
    const Tin* __restrict__ child, int64_t in_unit_stride, const Tr* __restrict__ Rall,
    float* __restrict__ out, int64_t out_unit_stride, int Hkv, int node_begin, int node_end,
    int b, float tau) {
  __shared__ float sR[kNRef][D];
  __shared__ float sX[kChunk][D + 4];
  __shared__ float sZ[kChunk][kNRef + 1];
  __shared__ float sW[kChunk];

  const int unit = blockIdx.y;
  const int per_wg = kChunk / b;
  const int node0 = node_begin + blockIdx.x * per_wg;
  if (node0 >= node_end) return;
  const int nn = min(per_wg, node_end - node0);
  const int rows = nn * b;

  stage_R<Tin, Tr, D>(sR, Rall + (int64_t)(unit % Hkv) * kNRef * D);
  stage_rows<Tin, D>(sX, child + unit * in_unit_stride + (int64_t)node0 * b * D, rows);
  __syncthreads();
  pool_scores<D>(sR, sX, sZ, rows, tau);
  __syncthreads();

  // softmax over the b children of each node, per reference query
  for (int i = threadIdx.x; i < nn * kNRef; i += kPoolThreads) {
    const int nd = i / kNRef, rf = i % kNRef;
    float mx = -INFINITY;
    for (int c = 0; c < b; ++c) mx = fmaxf(mx, sZ[nd * b + c][rf]);
    float sum = 0.f;
    for (int c = 0; c < b; ++c) sum += expf(sZ[nd * b + c][rf] - mx);
    for (int c = 0; c < b; ++c) sZ[nd * b + c][rf] = expf(sZ[nd * b + c][rf] - mx) / sum;
  }
  __syncthreads();
  // child weight = mean over the reference queries
  for (int r = threadIdx.x; r < rows; r += kPoolThreads) {
    float s = 0.f;
#pragma unroll
    for (int rf = 0; rf < kNRef; ++rf) s += sZ[r][rf];
    sW[r] = s * (1.f / kNRef);
  }
  __syncthreads();
  float* dst = out + unit * out_unit_stride + (int64_t)node0 * D;
  for (int i = threadIdx.x; i < nn * D; i += kPoolThreads) {
    const int nd = i / D, k = i % D;
    float acc = 0.f;
    for (int c = 0; c < b; ++c) acc = fmaf(sW[nd * b + c], sX[nd * b + c][k], acc);
    dst[(int64_t)nd * D + k] = acc;
  }
}

// b > 64: one workgroup per node, two passes over its children in chunks of 64:
// pass 1 finds each reference query's softmax max and normaliser, pass 2 recomputes the
// same scores and accumulates the weighted sum.
template <typename Tin, typename Tr, int D>
__global__ __launch_bounds__(kPoolThreads) void pool_large_kernel(
    const Tin* __restrict__ child, int64_t in_unit_stride, const Tr* __restrict__ Rall,
    float* __restrict__ out, int64_t out_unit_stride, int Hkv, int node_begin, int node_end,
    int b, float tau) {
  __shared__ float sR[kNRef][D];
  __shared__ float sX[kChunk][D + 4];
  __shared__ float sZ[kChunk][kNRef + 1];
  __shared__ float sW[kChunk];
  __shared__ float sMax[kNRef], sSum[kNRef];

  const int unit = blockIdx.y;
  const int node = node_begin + blockIdx.x;
  if (node >= node_end) return;
  const Tin* base = child + unit * in_unit_stride + (int64_t)node * b * D;

  stage_R<Tin, Tr, D>(sR, Rall + (int64_t)(unit % Hkv) * kNRef * D);
  if (threadIdx.x < kNRef) {
    sMax[threadIdx.x] = -INFINITY;
    sSum[threadIdx.x] = 0.f;
  }
  for (int c0 = 0; c0 < b; c0 += kChunk) {
    const int rows = min(kChunk, b - c0);
    __syncthreads();
    stage_rows<Tin, D>(sX, base + (int64_t)c0 * D, rows);
    __syncthreads();
    pool_scores<D>(sR, sX, sZ, rows, tau);
    __syncthreads();
    if (threadIdx.x < kNRef) {
      const int rf = threadIdx.x;
      float m = sMax[rf], s = sSum[rf];
      for (int c = 0; c < rows; ++c) {
        const float z = sZ[c][rf];
        const float mn = fmaxf(m, z);
        s = s * expf(m - mn) + expf(z - mn);
        m = mn;
      }
      sMax[rf] = m;
      sSum[rf] = s;
    }
  }
  float acc = 0.f;  // thread k < D owns output element k
  for (int c0 = 0; c0 < b; c0 += kChunk) {
    const int rows = min(kChunk, b - c0);
    __syncthreads();
    stage_rows<Tin, D>(sX, base + (int64_t)c0 * D, rows);
    __syncthreads();
    pool_scores<D>(sR, sX, sZ, rows, tau);
    __syncthreads();
    for (int r = threadIdx.x; r < rows; r += kPoolThreads) {
      float s = 0.f;
#pragma unroll
      for (int rf = 0; rf < kNRef; ++rf) s += expf(sZ[r][rf] - sMax[rf]) / sSum[rf];
      sW[r] = s * (1.f / kNRef);
    }
    __syncthreads();
    if (threadIdx.x < D)
      for (int c = 0; c < rows; ++c) acc = fmaf(sW[c], sX[c][threadIdx.x], acc);
  }
  if (threadIdx.x < D) out[unit * out_unit_stride + (int64_t)node * D + threadIdx.x] = acc;
}

template <typename Tin, typename Tr, int D>
hipError_t launch_pool_t(const void* child, int64_t in_unit_stride, const void* R, float* out,
                         int64_t out_unit_stride, int units, int Hkv, int node_begin,
                         int node_end, int b, hipStream_t s) {
  const float tau = 1.0f / sqrtf((float)D);
  const int nodes = node_end - node_begin;
  if (nodes <= 0) return hipSuccess;
  if (b <= kChunk) {
    const int per_wg = kChunk / b;
    dim3 grid((nodes + per_wg - 1) / per_wg, units);
    hipLaunchKernelGGL((pool_small_kernel<Tin, Tr, D>), grid, dim3(kPoolThreads), 0, s,
                       (const Tin*)child, in_unit_stride, (const Tr*)R, out, out_unit_stride,
                       Hkv, node_begin, node_end, b, tau);
  } else {
    dim3 grid(nodes, units);
    hipLaunchKernelGGL((pool_large_kernel<Tin, Tr, D>), grid, dim3(kPoolThreads), 0, s,
                       (const Tin*)child, in_unit_stride, (const Tr*)R, out, out_unit_stride,
                       Hkv, node_begin, node_end, b, tau);
  }
  return hipGetLastError();
}

template <typename Tin, typename Tr>
hipError_t launch_pool_d(int D, const void* child, int64_t in_unit_stride, const void* R,
                         float* out, int64_t out_unit_stride, int units, int Hkv,
                         int node_begin, int node_end, int b, hipStream_t s) {
  if (D == 64)
    return launch_pool_t<Tin, Tr, 64>(child, in_unit_stride, R, out, out_unit_stride, units, Hkv,
                                      node_begin, node_end, b, s);
  return launch_pool_t<Tin, Tr, 128>(child, in_unit_stride, R, out, out_unit_stride, units, Hkv,
                                     node_begin, node_end, b, s);
}

}  // namespace

hipError_t launch_pool_level(int dtype_in, const void* child, int64_t in_unit_stride,
                             const void* R, int dtype_r, float* out, int64_t out_unit_stride,
                             int units, int Hkv, int node_begin, int node_end, int b, int D,
                             hipStream_t s) {
  if (dtype_r == ZHA_BF16) {
    if (dtype_in == ZHA_BF16)
      return launch_pool_d<bf16_t, bf16_t>(D, child, in_unit_stride, R, out, out_unit_stride,
                                           units, Hkv, node_begin, node_end, b, s);
    return launch_pool_d<float, bf16_t>(D, child, in_unit_stride, R, out, out_unit_stride, units,
                                        Hkv, node_begin, node_end, b, s);
  }
  return launch_pool_d<float, float>(D, child, in_unit_stride, R, out, out_unit_stride, units,
                                     Hkv, node_begin, node_end, b, s);
}

}  // namespace zha
