// Sparse GQA decode over the gathered keys, with split-combine.
//
// Page 3, paragraph 1 (Le Fil IA / MarkTechPost): the full KV cache is kept and the
// tree only decides which keys each query reads; the first token is always kept.
// Attention is exact softmax attention at scale sigma = 1/sqrt(d) over each query
// head's selected tokens.
//
// Work list: the union, over a unit's members, of the kept level-1 nodes (ascending,
// with a member bitmask each), expanded to b contiguous tokens per node. Each K/V row is
// read once per unit and scored for every member; tokens outside a member's own set are
// masked. Tokens below `anchor` are skipped inside nodes and attended once, for every
// member, by split 0. The union token range is cut into `splits` equal pieces; each
// workgroup writes one (max, sum, weighted-V) partial per member and the last workgroup
// of a unit merges the partials in split order, so the result does not depend on which
// workgroup finishes last.

#include "zha_internal.h"

namespace zha {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;

template <typename T, int D>
__global__ __launch_bounds__(kDecThreads) void decode_valu_kernel(
    Geom geo, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ Q,
    LevelBufs l1, int anchor, int splits, float* __restrict__ part, uint32_t* __restrict__ done,
    float* __restrict__ O, float sigma) {
  constexpr int DPL = D / 64;  // dims per lane
  const int u = blockIdx.y, sp = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int Mu = members_of(geo, u);
  const int b = geo.b;
  const int ntok = (int)l1.count[u] * b;
  const int per = (ntok + splits - 1) / splits;
  const int t0 = min(sp * per, ntok), t1 = min(t0 + per, ntok);
  const int64_t row0 = (int64_t)bg_of(geo, u) * geo.Ncap;
  const T* Ku = K + row0 * D;
  const T* Vu = V + row0 * D;

  float q[kMaxMembers][DPL];
  float mrun[kMaxMembers], lrun[kMaxMembers], o[kMaxMembers][DPL];
#pragma unroll
  for (int m = 0; m < kMaxMembers; ++m) {
    mrun[m] = -INFINITY;
    lrun[m] = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      o[m][i] = 0.f;
      q[m][i] = (m < Mu) ? to_f32(Q[(int64_t)qh_of(geo, u, m) * D + lane * DPL + i]) : 0.f;
    }
  }
  const uint32_t full = (1u << Mu) - 1u;

  auto consume = [&](int tok, uint32_t mask) {
    float kx[DPL], vx[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      kx[i] = to_f32(Ku[(int64_t)tok * D + lane * DPL + i]);
      vx[i] = to_f32(Vu[(int64_t)tok * D + lane * DPL + i]);
    }
#pragma unroll
    for (int m = 0; m < kMaxMembers; ++m) {
      if (m >= Mu) continue;
      float v = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) v = fmaf(q[m][i], kx[i], v);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
      if (!((mask >> m) & 1u)) continue;
      const float s = sigma * v;
      const float mn = fmaxf(mrun[m], s);
      const float alpha = expf(mrun[m] - mn);
      const float beta = expf(s - mn);
      lrun[m] = lrun[m] * alpha + beta;
#pragma unroll
      for (int i = 0; i < DPL; ++i) o[m][i] = fmaf(o[m][i], alpha, beta * vx[i]);
      mrun[m] = mn;
    }
  };

  if (sp == 0 && wave == 0)
    for (int tok = 0; tok < anchor; ++tok) consume(tok, full);
  for (int i = t0 + wave; i < t1; i += kDecWaves) {
    const int nd = i / b, c = i % b;
    const int tok = (int)l1.nodes[u * l1.stride + nd] * b + c;
    if (tok < anchor) continue;
    consume(tok, l1.masks[u * l1.stride + nd]);
  }

  // merge the waves' states through LDS, in wave order
  __shared__ float sm[kDecWaves][kMaxMembers], sl[kDecWaves][kMaxMembers];
  __shared__ float so[kDecWaves][kMaxMembers][D];
#pragma unroll
  for (int m = 0; m < kMaxMembers; ++m) {
    if (lane == 0) {
      sm[wave][m] = mrun[m];
      sl[wave][m] = lrun[m];
    }
#pragma unroll
    for (int i = 0; i < DPL; ++i) so[wave][m][lane * DPL + i] = o[m][i];
  }
  __syncthreads();
  const int64_t pstride = (int64_t)(D + 2);
  float* pu = part + ((int64_t)u * splits + sp) * kMaxMembers * pstride;
  for (int idx = threadIdx.x; idx < Mu * D; idx += kDecThreads) {
    const int m = idx / D, k = idx % D;
    float M = -INFINITY;
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, sm[w][m]);
    float acc = 0.f, lsum = 0.f;
    if (M != -INFINITY) {
      for (int w = 0; w < kDecWaves; ++w) {
        if (sm[w][m] == -INFINITY) continue;
        const float f = expf(sm[w][m] - M);
        acc = fmaf(f, so[w][m][k], acc);
        lsum = fmaf(f, sl[w][m], lsum);
      }
    }
    pu[m * pstride + k] = acc;
    if (k == 0) {
      pu[m * pstride + D] = M;
      pu[m * pstride + D + 1] = lsum;
    }
  }

  // last workgroup of the unit combines every split, in split order
  __threadfence();
  __syncthreads();
  __shared__ uint32_t last;
  if (threadIdx.x == 0) last = (atomicAdd(&done[u], 1u) == (uint32_t)splits - 1u) ? 1u : 0u;
  __syncthreads();
  if (!last) return;
  __threadfence();
  const float* pall = part + (int64_t)u * splits * kMaxMembers * pstride;
  for (int idx = threadIdx.x; idx < Mu * D; idx += kDecThreads) {
    const int m = idx / D, k = idx % D;
    float M = -INFINITY;
    for (int s2 = 0; s2 < splits; ++s2) {
      const float ms = __hip_atomic_load(&pall[(s2 * kMaxMembers + m) * pstride + D],
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      M = fmaxf(M, ms);
    }
    float acc = 0.f, lsum = 0.f;
    for (int s2 = 0; s2 < splits; ++s2) {
      const float* ps = pall + (s2 * kMaxMembers + m) * pstride;
      const float ms = __hip_atomic_load(&ps[D], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (ms == -INFINITY) continue;
      const float f = expf(ms - M);
      acc = fmaf(f, __hip_atomic_load(&ps[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), acc);
      lsum = fmaf(f, __hip_atomic_load(&ps[D + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                  lsum);
    }
    O[(int64_t)qh_of(geo, u, m) * D + k] = acc / lsum;
  }
  if (threadIdx.x == 0) done[u] = 0u;
}

template <typename T>
hipError_t launch_decode_t(const Geom& geo, const void* K, const void* V, const void* Q,
                           const LevelBufs& l1, int anchor, int splits, float* partials,
                           uint32_t* done_dec, float* O, hipStream_t s) {
  dim3 grid(splits, geo.U);
  const float sigma = 1.0f / sqrtf((float)geo.D);
  if (geo.D == 64)
    hipLaunchKernelGGL((decode_valu_kernel<T, 64>), grid, dim3(kDecThreads), 0, s, geo,
                       (const T*)K, (const T*)V, (const T*)Q, l1, anchor, splits, partials,
                       done_dec, O, sigma);
  else
    hipLaunchKernelGGL((decode_valu_kernel<T, 128>), grid, dim3(kDecThreads), 0, s, geo,
                       (const T*)K, (const T*)V, (const T*)Q, l1, anchor, splits, partials,
                       done_dec, O, sigma);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const Geom& geo, int dtype, const void* K, const void* V,
                         const void* Q, const LevelBufs& l1, int anchor, int splits,
                         float* partials, uint32_t* done_dec, float* O, hipStream_t s) {
  if (dtype == ZHA_BF16)
    return launch_decode_t<bf16_t>(geo, K, V, Q, l1, anchor, splits, partials, done_dec, O, s);
  return launch_decode_t<float>(geo, K, V, Q, l1, anchor, splits, partials, done_dec, O, s);
}

}  // namespace zha
