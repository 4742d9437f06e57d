// Tree search: score a level's frontier, keep the smallest top-p set, expand.
//
// Page 3, paragraph 1 (Le Fil IA / MarkTechPost): a query evaluates the top nodes, keeps
// the smallest set covering a fraction p of the estimated attention mass, then expands
// only those branches down to the raw KV entries. Readings: the node score is
// sigma * q . X (sigma = 1/sqrt(d)); the estimated mass is the softmax of the scores over
// the current frontier; the same rule runs at every level on the children of the nodes
// kept one level up; order is descending score, ties by ascending node id; the cut is
// the first prefix whose cumulative mass is >= p.
//
// GQA: the members of a unit (the query heads, and queries, that read one KV head) share
// one union frontier per level, so each summary row is read once and scored for every
// member. Each member then selects over its own sub-frontier.

#include "zha_internal.h"

namespace zha {
namespace {

constexpr int kScoreThreads = 256;
constexpr int kScoreEntries = 256;  // frontier entries per workgroup

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kBuckets = 2048;
constexpr int kCand = 2048;
constexpr float kMassScale = 4398046511104.0f;  // 2^42: fixed-point scale of a node mass
constexpr float kMaxSpread = 32.0f;             // exp(-32) * 2^42 < 1: lower masses are 0

// node id of frontier entry k: the top level's frontier is every node; below, entry k
// is child k % b of the (k / b)-th node the level above kept (pnodes: that unit's list)
__device__ __forceinline__ uint32_t frontier_node(const uint32_t* pnodes, int k, int b) {
  if (!pnodes) return (uint32_t)k;
  return pnodes[k / b] * (uint32_t)b + (uint32_t)(k % b);
}

template <int D, typename Tq>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(
    Geom geo, const float* __restrict__ X, int64_t X_unit_stride, const Tq* __restrict__ Q,
    LevelBufs parent, int has_parent, int n_top, float* __restrict__ S, int64_t S_stride,
    LevelBufs cur, float sigma) {
  constexpr int LPR = D / 4;       // lanes per row (4 floats per lane)
  constexpr int RPW = 64 / LPR;    // rows per wave per step
  const int u = blockIdx.y;
  const int F = has_parent ? geo.b * (int)parent.count[u] : n_top;
  const int k_wg = blockIdx.x * kScoreEntries;
  if (k_wg >= F) return;
  const int Mu = members_of(geo, u);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, li = lane % LPR;

  float q[kMaxMembers][4];
#pragma unroll
  for (int m = 0; m < kMaxMembers; ++m) {
    if (m < Mu) {
      const Tq* qp = Q + (int64_t)qh_of(geo, u, m) * D + li * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) q[m][i] = to_f32(qp[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) q[m][i] = 0.f;
    }
  }
  const float* Xu = X + (int64_t)bg_of(geo, u) * X_unit_stride;
  const uint32_t full = (Mu >= 32) ? 0xffffffffu : ((1u << Mu) - 1u);
  const uint32_t* pnodes = has_parent ? parent.nodes + u * parent.stride : nullptr;
  constexpr int kPerWave = kScoreEntries / (kScoreThreads / 64);

  for (int e = 0; e < kPerWave; e += RPW) {
    const int k = k_wg + wave * kPerWave + e + sub;
    const bool valid = k < F;
    uint32_t mask = 0;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) {
      const uint32_t node = frontier_node(pnodes, k, geo.b);
      mask = has_parent ? parent.masks[u * parent.stride + k / geo.b] : full;
      x = *reinterpret_cast<const float4*>(Xu + (int64_t)node * D + li * 4);
    }
    float mine = 0.f;
#pragma unroll
    for (int m = 0; m < kMaxMembers; ++m) {
      float v = q[m][0] * x.x;
      v = fmaf(q[m][1], x.y, v);
      v = fmaf(q[m][2], x.z, v);
      v = fmaf(q[m][3], x.w, v);
#pragma unroll
      for (int off = LPR / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
      if (m == li) mine = v;
    }
    if (valid) {
      if (li == 0) cur.keep[u * cur.stride + k] = 0u;
      if (li < Mu && ((mask >> li) & 1u)) {
        // + 0.0f turns a -0 score into +0 so float and bit orders agree
        S[(int64_t)qh_of(geo, u, li) * S_stride + k] = sigma * mine + 0.0f;
      }
    }
  }
}

// ------------------------------------------------------------------------- selection

__device__ __forceinline__ uint32_t ord_of(float s) {
  const uint32_t v = __float_as_uint(s);
  return (v & 0x80000000u) ? ~v : (v | 0x80000000u);
}
__device__ __forceinline__ float float_of_ord(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
// rank key: larger = earlier in (score desc, index asc)
__device__ __forceinline__ uint64_t rank_key(float s, uint32_t k) {
  return ((uint64_t)ord_of(s) << 32) | (uint64_t)(0xffffffffu - k);
}
__device__ __forceinline__ uint64_t mass_fixed(float s, float smax) {
  return (uint64_t)(expf(s - smax) * kMassScale);
}
// bucket 0 holds the highest scores; t * scale stays within [0, kBuckets] because
// t is clamped to the spread that defines the scale
__device__ __forceinline__ int bucket_of(float s, float smax, float scale, float spread) {
  const float t = fminf(smax - s, spread);
  const int b = (int)(t * scale);
  return b < kBuckets - 1 ? b : kBuckets - 1;
}

// ceil(p * Z) exactly, for 0 < p < 1 (p = mant * 2^-sh, mant < 2^24, sh >= 24)
__device__ uint64_t ceil_mul_p(float p, uint64_t Z) {
  int e;
  const float f = frexpf(p, &e);
  const uint64_t mant = (uint64_t)(f * 16777216.0f);
  const int sh = 24 - e;
  const uint64_t lo = mant * Z, hi = __umul64hi(mant, Z);
  uint64_t q;
  bool rem;
  if (sh >= 128) {
    q = 0;
    rem = (lo | hi) != 0;
  } else if (sh >= 64) {
    const int s2 = sh - 64;
    q = s2 ? (hi >> s2) : hi;
    rem = lo != 0 || (s2 && (hi & ((1ull << s2) - 1)));
  } else {
    q = (lo >> sh) | (hi << (64 - sh));
    rem = (lo & ((1ull << sh) - 1)) != 0;
  }
  return q + (rem ? 1 : 0);
}

__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v, int d) {
  const uint32_t lo = __shfl_up((uint32_t)v, d, 64), hi = __shfl_up((uint32_t)(v >> 32), d, 64);
  return ((uint64_t)hi << 32) | lo;
}

// inclusive scan across one wave
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t o = shfl_up_u64(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

struct SelShared {
  unsigned long long hm[kBuckets];
  uint32_t hc[kBuckets];
  unsigned long long cand[kCand];
  float red_f[2][kSelWaves];
  uint32_t red_u[kSelWaves];
  uint32_t wave_cnt[kSelWaves];
  uint32_t tile_nodes[kSelThreads];
  unsigned long long scalar_u64[4];
  uint32_t scalar_u32[8];
  float scalar_f[4];
};

// Block-wide exclusive rank of `flag` in thread order; returns rank, *total = count.
__device__ __forceinline__ uint32_t block_rank(bool flag, uint32_t* wave_cnt, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t bal = __ballot(flag);
  const uint32_t in_wave = __popcll(bal & ((1ull << lane) - 1ull));
  __syncthreads();
  if (lane == 0) wave_cnt[wave] = __popcll(bal);
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const uint32_t c = wave_cnt[w];
    before += (w < wave) ? c : 0;
    tot += c;
  }
  *total = tot;
  return before + in_wave;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    Geom geo, int level, const float* __restrict__ S, int64_t S_stride, LevelBufs parent,
    int has_parent, int n_top, LevelBufs cur, float p, int anchor, int32_t* __restrict__ sel_idx,
    int64_t cap, int32_t* __restrict__ sel_count, int32_t* __restrict__ lvl_kept) {
  __shared__ SelShared sh;
  const int qh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int u, m;
  unit_member_of(geo, qh, &u, &m);
  const int b = geo.b;
  const int F = has_parent ? b * (int)parent.count[u] : n_top;
  const float* Sq = S + (int64_t)qh * S_stride;
  const uint32_t* pmask = has_parent ? parent.masks + u * parent.stride : nullptr;
  const uint32_t* pnodes = has_parent ? parent.nodes + u * parent.stride : nullptr;
  auto member = [&](int k) -> bool { return !pmask || ((pmask[k / b] >> m) & 1u); };

  if (tid == 0) {
    sh.scalar_u32[1] = 0u;
    sh.scalar_u64[0] = 0ull;
    sh.scalar_u64[1] = 0ull;
    sh.scalar_u64[2] = ~0ull;
  }
  // pass 0: max, min over the member's frontier
  float mx = -INFINITY, mn = INFINITY;
  for (int k = tid; k < F; k += kSelThreads) {
    if (member(k)) {
      const float s = Sq[k];
      mx = fmaxf(mx, s);
      mn = fminf(mn, s);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    mn = fminf(mn, __shfl_xor(mn, off, 64));
  }
  if (lane == 0) {
    sh.red_f[0][wave] = mx;
    sh.red_f[1][wave] = mn;
  }
  __syncthreads();
  mx = sh.red_f[0][0];
  mn = sh.red_f[1][0];
#pragma unroll
  for (int w = 1; w < kSelWaves; ++w) {
    mx = fmaxf(mx, sh.red_f[0][w]);
    mn = fminf(mn, sh.red_f[1][w]);
  }

  const bool keep_all = !(p < 1.0f);
  float s_cut = -INFINITY;
  uint32_t k_cut = 0xffffffffu;
  if (!keep_all) {
    const float spread = fminf(mx - mn, kMaxSpread);
    const float scale = spread > 0.f ? (float)kBuckets / spread : 0.f;
    for (int i = tid; i < kBuckets; i += kSelThreads) {
      sh.hm[i] = 0ull;
      sh.hc[i] = 0u;
    }
    if (tid == 0) sh.scalar_u32[0] = 0u;
    __syncthreads();
    // pass 1: fixed-point mass histogram over score buckets (bucket 0 = highest scores)
    for (int k = tid; k < F; k += kSelThreads) {
      if (member(k)) {
        const float s = Sq[k];
        const int bk = bucket_of(s, mx, scale, spread);
        atomicAdd(&sh.hm[bk], (unsigned long long)mass_fixed(s, mx));
        atomicAdd(&sh.hc[bk], 1u);
      }
    }
    __syncthreads();
    // wave 0: total mass, target, and the bucket where the cumulative mass reaches it
    if (wave == 0) {
      constexpr int per = kBuckets / 64;
      uint64_t loc = 0;
      for (int i = 0; i < per; ++i) loc += sh.hm[lane * per + i];
      const uint64_t incl = wave_incl_scan_u64(loc, lane);
      const uint64_t Z = __shfl(incl, 63, 64);
      const uint64_t T = ceil_mul_p(p, Z);
      const uint64_t excl = incl - loc;
      if (excl < T && incl >= T) {
        uint64_t run = excl;
        for (int i = 0; i < per; ++i) {
          const uint64_t nxt = run + sh.hm[lane * per + i];
          if (nxt >= T) {
            sh.scalar_u32[1] = lane * per + i;  // B*
            sh.scalar_u64[0] = run;             // mass strictly before B*
            break;
          }
          run = nxt;
        }
      }
      if (lane == 0) sh.scalar_u64[1] = T;
    }
    __syncthreads();
    const int bstar = (int)sh.scalar_u32[1];
    const uint64_t before = sh.scalar_u64[0];
    const uint64_t T = sh.scalar_u64[1];
    const uint32_t nb = sh.hc[bstar];
    if (nb <= (uint32_t)kCand) {
      // gather the boundary bucket, sort it by rank key, scan its masses
      for (int k = tid; k < F; k += kSelThreads) {
        if (member(k)) {
          const float s = Sq[k];
          if (bucket_of(s, mx, scale, spread) == bstar) {
            const uint32_t slot = atomicAdd(&sh.scalar_u32[0], 1u);
            sh.cand[slot] = rank_key(s, (uint32_t)k);
          }
        }
      }
      __syncthreads();
      int P2 = 1;
      while (P2 < (int)nb) P2 <<= 1;
      for (int i = nb + tid; i < P2; i += kSelThreads) sh.cand[i] = 0ull;
      __syncthreads();
      for (int size = 2; size <= P2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          for (int i = tid; i < P2; i += kSelThreads) {
            const int j = i ^ stride;
            if (j > i) {
              const unsigned long long a = sh.cand[i], c = sh.cand[j];
              const bool desc = (i & size) == 0;  // descending blocks give a descending result
              if (desc ? (a < c) : (a > c)) {
                sh.cand[i] = c;
                sh.cand[j] = a;
              }
            }
          }
          __syncthreads();
        }
      }
      if (wave == 0) {
        const int per = (P2 + 63) / 64;
        uint64_t loc = 0;
        for (int i = 0; i < per; ++i) {
          const int idx = lane * per + i;
          if (idx < (int)nb) loc += mass_fixed(float_of_ord((uint32_t)(sh.cand[idx] >> 32)), mx);
        }
        const uint64_t incl = wave_incl_scan_u64(loc, lane) + before;
        const uint64_t excl = incl - loc;
        if (excl < T && incl >= T) {
          uint64_t run = excl;
          for (int i = 0; i < per; ++i) {
            const int idx = lane * per + i;
            if (idx >= (int)nb) break;
            const uint64_t key = sh.cand[idx];
            run += mass_fixed(float_of_ord((uint32_t)(key >> 32)), mx);
            if (run >= T) {
              sh.scalar_u64[2] = key;
              break;
            }
          }
        }
      }
      __syncthreads();
    } else {
      // boundary bucket too large to sort: exact MSD radix select on the 64-bit rank
      // key, restricted to the boundary bucket, 8 bits per pass
      uint64_t prefix = 0, pmask_bits = 0, need = T - before;
      for (int shift = 56; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kSelThreads) sh.hm[i] = 0ull;
        __syncthreads();
        for (int k = tid; k < F; k += kSelThreads) {
          if (member(k)) {
            const float s = Sq[k];
            if (bucket_of(s, mx, scale, spread) != bstar) continue;
            const uint64_t key = rank_key(s, (uint32_t)k);
            if ((key & pmask_bits) != prefix) continue;
            atomicAdd(&sh.hm[(key >> shift) & 255u], (unsigned long long)mass_fixed(s, mx));
          }
        }
        __syncthreads();
        if (tid == 0) {
          uint64_t run = 0;
          int dsel = 0;
          for (int dg = 255; dg >= 0; --dg) {
            if (run + sh.hm[dg] >= need) {
              dsel = dg;
              break;
            }
            run += sh.hm[dg];
          }
          sh.scalar_u64[3] = ((uint64_t)dsel << 32) | 0u;
          sh.scalar_u64[2] = run;
        }
        __syncthreads();
        const uint64_t dsel = sh.scalar_u64[3] >> 32;
        need -= sh.scalar_u64[2];
        prefix |= dsel << shift;
        pmask_bits |= 255ull << shift;
        __syncthreads();
      }
      if (tid == 0) sh.scalar_u64[2] = prefix;
      __syncthreads();
    }
    const uint64_t key = sh.scalar_u64[2];
    s_cut = float_of_ord((uint32_t)(key >> 32));
    k_cut = 0xffffffffu - (uint32_t)key;
  }
  auto kept_at = [&](int k) -> bool {
    if (!member(k)) return false;
    if (keep_all) return true;
    const float s = Sq[k];
    return s > s_cut || (s == s_cut && (uint32_t)k <= k_cut);
  };

  // anchor overlap: kept level-1 tokens below `anchor` (they can only sit in the first
  // ceil(anchor / b) frontier entries, since node ids are distinct and ascending)
  int dup = 0;
  if (level == 1 && tid == 0) {
    const int lim = min(F, (anchor + b - 1) / b);
    for (int k = 0; k < lim; ++k) {
      if (kept_at(k)) {
        const int node = (int)frontier_node(pnodes, k, b);
        if (node * b < anchor) dup += min(b, anchor - node * b);
      }
    }
    sh.scalar_u32[2] = (uint32_t)dup;
  }
  __syncthreads();
  dup = (int)sh.scalar_u32[2];
  int32_t* sel = sel_idx ? sel_idx + (int64_t)qh * cap : nullptr;
  if (level == 1 && sel)
    for (int i = tid; i < anchor; i += kSelThreads) sel[i] = i;

  // emit: mark kept entries in the unit's keep masks; at level 1 write the token list
  uint32_t running = 0;
  for (int k0 = 0; k0 < F; k0 += kSelThreads) {
    const int k = k0 + tid;
    const bool kept = k < F && kept_at(k);
    if (kept) atomicOr(&cur.keep[u * cur.stride + k], 1u << m);
    uint32_t tile_total;
    const uint32_t r = block_rank(kept, sh.wave_cnt, &tile_total);
    if (level == 1 && sel) {
      if (kept) sh.tile_nodes[r] = frontier_node(pnodes, k, b);
      __syncthreads();
      const int ntok = (int)tile_total * b;
      for (int i = tid; i < ntok; i += kSelThreads) {
        const int rr = i / b, c = i % b;
        const int tok = (int)sh.tile_nodes[rr] * b + c;
        if (tok >= anchor) sel[anchor + (int64_t)(running + rr) * b + c - dup] = tok;
      }
    }
    running += tile_total;
  }
  if (tid == 0) {
    lvl_kept[(int64_t)qh * (geo.L + 1) + level] = (int32_t)running;
    if (level == 1) sel_count[qh] = anchor + (int32_t)running * b - dup;
  }

  // the last member of the unit to finish compacts the union keep masks into the
  // ascending list of kept nodes for the next level (or for the decode at level 1)
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = atomicAdd(&cur.done[u], 1u);
    sh.scalar_u32[3] = (prev == (uint32_t)members_of(geo, u) - 1u) ? 1u : 0u;
  }
  __syncthreads();
  if (sh.scalar_u32[3] == 0u) return;
  __threadfence();
  uint32_t out = 0;
  for (int k0 = 0; k0 < F; k0 += kSelThreads) {
    const int k = k0 + tid;
    uint32_t msk = 0;
    if (k < F)
      msk = __hip_atomic_load(&cur.keep[u * cur.stride + k], __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
    uint32_t tile_total;
    const uint32_t r = block_rank(msk != 0u, sh.wave_cnt, &tile_total);
    if (msk) {
      cur.nodes[u * cur.stride + out + r] = frontier_node(pnodes, k, b);
      cur.masks[u * cur.stride + out + r] = msk;
    }
    out += tile_total;
  }
  if (tid == 0) {
    cur.count[u] = out;
    cur.done[u] = 0u;
  }
}

__global__ void init_kernel(uint32_t* done_all, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    done_all[i] = 0u;
}

}  // namespace

hipError_t launch_attend_init(uint32_t* done_all, int n, hipStream_t s) {
  hipLaunchKernelGGL(init_kernel, dim3(1), dim3(256), 0, s, done_all, n);
  return hipGetLastError();
}

hipError_t launch_score(const Geom& geo, int level, const float* X, int64_t X_unit_stride,
                        const void* Q, int dtype, const LevelBufs* parent, int n_top, float* S,
                        int64_t S_stride, const LevelBufs& cur, hipStream_t s) {
  (void)level;
  const int cap_entries = parent ? (int)cur.stride : n_top;
  dim3 grid((cap_entries + kScoreEntries - 1) / kScoreEntries, geo.U);
  const float sigma = 1.0f / sqrtf((float)geo.D);
  LevelBufs par = parent ? *parent : LevelBufs{};
  const int hp = parent ? 1 : 0;
  if (geo.D == 64) {
    if (dtype == ZHA_BF16)
      hipLaunchKernelGGL((score_kernel<64, bf16_t>), grid, dim3(kScoreThreads), 0, s, geo, X,
                         X_unit_stride, (const bf16_t*)Q, par, hp, n_top, S, S_stride, cur, sigma);
    else
      hipLaunchKernelGGL((score_kernel<64, float>), grid, dim3(kScoreThreads), 0, s, geo, X,
                         X_unit_stride, (const float*)Q, par, hp, n_top, S, S_stride, cur, sigma);
  } else {
    if (dtype == ZHA_BF16)
      hipLaunchKernelGGL((score_kernel<128, bf16_t>), grid, dim3(kScoreThreads), 0, s, geo, X,
                         X_unit_stride, (const bf16_t*)Q, par, hp, n_top, S, S_stride, cur, sigma);
    else
      hipLaunchKernelGGL((score_kernel<128, float>), grid, dim3(kScoreThreads), 0, s, geo, X,
                         X_unit_stride, (const float*)Q, par, hp, n_top, S, S_stride, cur, sigma);
  }
  return hipGetLastError();
}

hipError_t launch_select(const Geom& geo, int level, const float* S, int64_t S_stride,
                         const LevelBufs* parent, int n_top, const LevelBufs& cur, float p,
                         int anchor, int32_t* sel_idx, int64_t cap, int32_t* sel_count,
                         int32_t* lvl_kept, hipStream_t s) {
  LevelBufs par = parent ? *parent : LevelBufs{};
  const int QH = geo.B * geo.T * geo.Hq;
  hipLaunchKernelGGL(select_kernel, dim3(QH), dim3(kSelThreads), 0, s, geo, level, S, S_stride,
                     par, parent ? 1 : 0, n_top, cur, p, anchor, sel_idx, cap, sel_count,
                     lvl_kept);
  return hipGetLastError();
}

}  // namespace zha
