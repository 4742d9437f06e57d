// The FP4 router's summary keys (page 3, paragraph 4 of the Le Fil IA ZHA article: a
// variant of the router in FP4 was also tested): the float32 pyramid rows encoded as
// MXFP4 (OCP Microscaling Formats v1.0), one launch for every level of a call.
//
// Work split: a row of d floats is taken by d / 8 lanes, eight consecutive elements each
// (two 16-byte loads); the four lanes of a 32-element block agree on its largest
// magnitude by two shuffles, then each lane writes its eight codes as one 32-bit word and
// the block's first lane writes the scale byte. Rows of one level are consecutive, so a
// workgroup reads 16 (d = 128) or 32 (d = 64) whole rows and writes their codes as one
// contiguous run. HBM-bound: 4d bytes read and d / 2 + d / 32 bytes written per row.

#include "zha_internal.h"
#include "zha_mxfp4.h"

namespace zha {
namespace {

constexpr int kRouterThreads = 256;

template <int D>
__global__ __launch_bounds__(kRouterThreads) void router_encode_kernel(RouterJob job) {
  constexpr int LPR = D / 8;                 // lanes per row
  constexpr int RPW = kRouterThreads / LPR;  // rows per workgroup
  const int u = blockIdx.y;
  int li = 0;  // the job's level: the last whose first workgroup is at or before this one
  for (int i = 1; i < job.n; ++i)
    if ((int)blockIdx.x >= job.wg0[i]) li = i;
  const int row = job.row0[li] + ((int)blockIdx.x - job.wg0[li]) * RPW + (int)threadIdx.x / LPR;
  const int sub = (int)threadIdx.x % LPR;
  const bool ok = row < job.row1[li];
  // rows past the level's end read its first row (in bounds) and store nothing
  const int64_t r = (int64_t)u * job.rows_cap[li] + (ok ? row : job.row0[li]);
  const float4* src = reinterpret_cast<const float4*>(job.src[li] + r * D + 8 * sub);
  const float4 a = src[0], c = src[1];
  const float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const uint32_t sb = mx_scale_byte(amax);
  const uint32_t w = e2m1_pack8(x, mx_inv_scale(sb));
  if (ok) {
    reinterpret_cast<uint32_t*>(job.codes[li] + r * (D / 2))[sub] = w;
    if ((sub & 3) == 0) job.scales[li][r * (D / kMxBlock) + sub / 4] = (uint8_t)sb;
  }
}

}  // namespace

int router_rows_per_workgroup(int D) { return kRouterThreads / (D / 8); }

hipError_t launch_router_encode(const RouterJob& job, int units, int D, int workgroups,
                                hipStream_t s) {
  if (job.n < 1 || workgroups < 1) return hipSuccess;
  const dim3 grid(workgroups, units);
  if (D == 64)
    hipLaunchKernelGGL(router_encode_kernel<64>, grid, dim3(kRouterThreads), 0, s, job);
  else
    hipLaunchKernelGGL(router_encode_kernel<128>, grid, dim3(kRouterThreads), 0, s, job);
  return hipGetLastError();
}

}  // namespace zha
