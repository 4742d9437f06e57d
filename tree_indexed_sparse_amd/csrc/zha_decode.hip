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
// masked. Tokens below `anchor` are skipped inside nodes and attended once, by split 0,
// for every member that sees them. Each member's tail (the tokens it sees after its last
// complete top node and its anchor, or every token it sees for dense attention) is
// covered by one range that follows the list, masked per member. Without query positions
// every member sees all N tokens and these ranges are the same for all of them.
// The work range (list tokens, then tail) is cut into `splits` equal pieces; each
// workgroup writes one (max, sum, weighted-V) partial per member, and a separate combine
// launch merges a unit's partials in a fixed order, so the result does not depend on the
// order in which workgroups run.

#include "zha_internal.h"

namespace zha {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kNodeChunk = 2048;  // union-list entries staged in LDS at a time

// What the members of a unit see: anchor tokens [0, anc[m]), tail [tlo[m], vis[m]).
// Written by threads 0 .. kMaxMembers - 1; read after a barrier.
struct UnitRanges {
  int anc[kMaxMembers], tlo[kMaxMembers], vis[kMaxMembers];
};

__device__ __forceinline__ void unit_ranges_fill(const Geom& geo, int u, int Mu, int has_list,
                                                 int anchor, UnitRanges& r) {
  const int m = threadIdx.x;
  if (m >= kMaxMembers) return;
  int vis = 0, an = 0, tlo = 0;
  if (m < Mu) {
    vis = head_vis(geo, qh_of(geo, u, m));
    an = min(anchor, vis);
    tlo = has_list ? max((vis / geo.top_span) * geo.top_span, an) : 0;
  }
  r.anc[m] = an;
  r.tlo[m] = tlo;
  r.vis[m] = vis;
}

// The unit's tail span [*lo, *lo + *n) (the members' tails together) and anchor span.
__device__ __forceinline__ void unit_spans(const UnitRanges& r, int Mu, int* lo, int* n,
                                           int* anc) {
  int a = 0, l = 0x7fffffff, h = 0;
  for (int m = 0; m < Mu; ++m) {
    a = max(a, r.anc[m]);
    if (r.vis[m] > r.tlo[m]) {
      l = min(l, r.tlo[m]);
      h = max(h, r.vis[m]);
    }
  }
  *anc = a;
  *lo = h > 0 ? l : 0;
  *n = h > 0 ? h - l : 0;
}

// Members for whom token `tok` is an anchor token / a tail token.
__device__ __forceinline__ uint32_t anchor_members(const UnitRanges& r, int Mu, int tok) {
  uint32_t mk = 0u;
  for (int m = 0; m < Mu; ++m) mk |= (uint32_t)(tok < r.anc[m]) << m;
  return mk;
}
__device__ __forceinline__ uint32_t tail_members(const UnitRanges& r, int Mu, int tok) {
  uint32_t mk = 0u;
  for (int m = 0; m < Mu; ++m) mk |= (uint32_t)(tok >= r.tlo[m] && tok < r.vis[m]) << m;
  return mk;
}

// Merge the per-wave states (sm, sl: [wave][member], so: [wave][member][D], in LDS) into
// this split's partial (max, sum, sum of p * v per member). Every thread calls this.
template <int D>
__device__ void write_partial(int u, int sp, int splits, int Mu, const float* sm, const float* sl,
                              const float* so, float* __restrict__ part) {
  const int64_t pstride = (int64_t)(D + 2);
  float* pu = part + ((int64_t)u * splits + sp) * kMaxMembers * pstride;
  for (int idx = threadIdx.x; idx < Mu * D; idx += kDecThreads) {
    const int m = idx / D, k = idx % D;
    float M = -INFINITY;
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, sm[w * kMaxMembers + m]);
    float acc = 0.f, lsum = 0.f;
    if (M != -INFINITY) {
      for (int w = 0; w < kDecWaves; ++w) {
        const float mw = sm[w * kMaxMembers + m];
        if (mw == -INFINITY) continue;
        const float f = expf(mw - M);
        acc = fmaf(f, so[(w * kMaxMembers + m) * D + k], acc);
        lsum = fmaf(f, sl[w * kMaxMembers + m], lsum);
      }
    }
    pu[m * pstride + k] = acc;
    if (k == 0) {
      pu[m * pstride + D] = M;
      pu[m * pstride + D + 1] = lsum;
    }
  }
}

// One workgroup per (unit, member): merge the member's partials of every split into its
// output row, in a fixed order (wave 0 forms the split weights; thread (split lane, column
// pair) accumulates splits lane, lane + SL, ...; the split lanes are then added in order),
// so the result does not depend on the order in which workgroups run. Runs after the
// decode launch, which orders it.
constexpr int kCombThreads = 256;

template <int D>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(Geom geo, int splits,
                                                               const float* __restrict__ part,
                                                               float* __restrict__ O) {
  constexpr int DP = D / 2;                // float2 columns per partial row
  constexpr int SL = kCombThreads / DP;    // split lanes
  __shared__ float sw[kMaxSplits];
  __shared__ float2 sacc[SL][DP];
  const int u = blockIdx.x, m = blockIdx.y;
  if (m >= members_of(geo, u)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t pstride = (int64_t)(D + 2);  // rows are 8-byte aligned: float2 loads
  const int64_t sstride = kMaxMembers * pstride;
  const float* pm = part + ((int64_t)u * splits * kMaxMembers + m) * pstride;
  if (tid < 64) {
    float M = -INFINITY;
    for (int s2 = lane; s2 < splits; s2 += 64) M = fmaxf(M, pm[s2 * sstride + D]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    float L = 0.f;
    for (int s2 = lane; s2 < splits; s2 += 64) {
      const float w = pm[s2 * sstride + D];
      if (w != -INFINITY) L = fmaf(expf(w - M), pm[s2 * sstride + D + 1], L);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off, 64);
    for (int s2 = lane; s2 < splits; s2 += 64) {
      const float w = pm[s2 * sstride + D];
      sw[s2] = (w == -INFINITY) ? 0.f : expf(w - M) / L;
    }
  }
  __syncthreads();
  const int col = tid % DP, sl = tid / DP;
  float ax = 0.f, ay = 0.f;
#pragma unroll 8
  for (int s2 = sl; s2 < splits; s2 += SL) {
    const float2 v = *reinterpret_cast<const float2*>(pm + s2 * sstride + 2 * col);
    ax = fmaf(sw[s2], v.x, ax);
    ay = fmaf(sw[s2], v.y, ay);
  }
  sacc[sl][col] = make_float2(ax, ay);
  __syncthreads();
  if (sl == 0) {
    float2 r = sacc[0][col];
#pragma unroll
    for (int j = 1; j < SL; ++j) {
      r.x += sacc[j][col].x;
      r.y += sacc[j][col].y;
    }
    *reinterpret_cast<float2*>(O + (int64_t)qh_of(geo, u, m) * D + 2 * col) = r;
  }
}

// Split sp of `splits` over ntok work items: boundaries on multiples of `align`, the
// pieces as equal as that allows (no short or empty last piece).
__device__ __forceinline__ void split_range(int ntok, int splits, int sp, int align, int* t0,
                                            int* t1) {
  const int64_t pieces = (ntok + align - 1) / align;
  *t0 = min((int)(sp * pieces / splits) * align, ntok);
  *t1 = min((int)((sp + 1) * pieces / splits) * align, ntok);
}

// float32 inputs: lanes across head dims, one token at a time per wave.
template <typename T, int D>
__global__ __launch_bounds__(kDecThreads) void decode_valu_kernel(
    Geom geo, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ Q,
    LevelBufs l1, int has_list, int anchor, int splits, float* __restrict__ part,
    float sigma) {
  constexpr int DPL = D / 64;  // dims per lane
  __shared__ UnitRanges rg;
  const int u = blockIdx.y, sp = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int Mu = members_of(geo, u);
  const int b = geo.b;
  const int nnode = has_list ? (int)l1.count[u] * b : 0;  // work items from the list
  unit_ranges_fill(geo, u, Mu, has_list, anchor, rg);
  __syncthreads();
  int tail_lo, n_tail, anc_u;
  unit_spans(rg, Mu, &tail_lo, &n_tail, &anc_u);
  int t0, t1;
  split_range(nnode + n_tail, splits, sp, 1, &t0, &t1);
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

  const uint32_t full = (1u << Mu) - 1u;  // without query positions: every member
  if (sp == 0 && wave == 0)
    for (int tok = 0; tok < anc_u; ++tok)
      consume(tok, geo.pos ? anchor_members(rg, Mu, tok) : full);
  for (int i = t0 + wave; i < t1; i += kDecWaves) {
    if (i >= nnode) {  // the tail: the members whose tail holds the token
      const int tok = tail_lo + (i - nnode);
      consume(tok, geo.pos ? tail_members(rg, Mu, tok) : full);
      continue;
    }
    const int nd = (int)geo.bdiv.div((uint32_t)i), c = i - nd * b;
    const int tok = (int)l1.nodes[u * l1.stride + nd] * b + c;
    if (tok < anchor) continue;
    consume(tok, l1.masks[u * l1.stride + nd]);
  }

  // merge the waves' states through LDS, in wave order
  __shared__ float sm[kDecWaves][kMaxMembers], sl[kDecWaves][kMaxMembers];
  __shared__ float so[kDecWaves * kMaxMembers * D];
#pragma unroll
  for (int m = 0; m < kMaxMembers; ++m) {
    if (lane == 0) {
      sm[wave][m] = mrun[m];
      sl[wave][m] = lrun[m];
    }
#pragma unroll
    for (int i = 0; i < DPL; ++i) so[(wave * kMaxMembers + m) * D + lane * DPL + i] = o[m][i];
  }
  __syncthreads();
  write_partial<D>(u, sp, splits, Mu, &sm[0][0], &sl[0][0], so, part);
}

// ------------------------------------------------------------------------------------
// bf16 inputs: matrix cores. Each wave walks 32-token tiles of the split's range.
//   S^T[token][member] = K . Q^T  with v_mfma_f32_16x16x32_bf16: A = 16 key rows (each lane
//     loads 16 contiguous bytes of its row straight from HBM), B = the members' queries,
//     held in registers for the whole kernel. Two 16-token halves per tile.
//   O^T[dim][member] += V^T . P^T: the probabilities stay in the lanes that produced them,
//     which is exactly the B-operand layout once token slots are numbered to match; V is
//     staged through a padded LDS tile and each lane reads one dword (two adjacent dims)
//     per token, feeding an even-dim and an odd-dim MFMA. P is split into bf16 hi + lo
//     parts (two MFMAs) so the product keeps about 16 mantissa bits; accumulation is fp32.
// Lane l: member = l % 16, group = l / 16. Softmax state per member is shared by the 4
// lanes of that member (one per group); the running sum is kept per lane and reduced at
// the end. The workgroup's slice of the union node list is staged in LDS, and each wave
// issues the loads of its next tile before computing the current one.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 32;

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint4 ld16(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// K and V rows are read once per call: non-temporal loads keep them from displacing
// reusable lines in the caches.
__device__ __forceinline__ uint4 ld16_stream(const bf16_t* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int D>
struct TileRegs {
  uint4 k[2][D / 32];
  uint4 v[kTile / (64 / (D / 8))];
};

template <int D>
__global__ __launch_bounds__(kDecThreads, 2) void decode_mfma_kernel(
    Geom geo, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ Q, LevelBufs l1, int has_list, int anchor,
    int splits, float* __restrict__ part, float sigma) {
  constexpr int KC = D / 32;          // 32-dim chunks: QK k-steps and PV column blocks
  constexpr int RW = D / 2 + 4;       // LDS row stride in dwords (padding spreads banks)
  constexpr int CH = D / 8;           // 16-byte chunks per row
  constexpr int RPI = 64 / CH;        // rows per wave-wide 16-byte load
  constexpr int NI = kTile / RPI;     // such loads per tile
  constexpr int VWORDS = kDecWaves * kTile * RW;
  constexpr int MWORDS = kDecWaves * kMaxMembers * (D + 2);
  __shared__ uint32_t smem[VWORDS > MWORDS ? VWORDS : MWORDS];
  __shared__ uint32_t s_nodes[kNodeChunk], s_masks[kNodeChunk];
  __shared__ __align__(16) int s_tt[kDecWaves * 2 * kTile];
  __shared__ __align__(16) uint32_t s_tm[kDecWaves * 2 * kTile];

  const int u = blockIdx.y, sp = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mem = lane & 15, grp = lane >> 4;
  const int Mu = members_of(geo, u);
  const int b = geo.b;
  const int ncount = has_list ? (int)l1.count[u] : 0;
  const int nnode = ncount * b;  // work items from the list; the tail follows them
  __shared__ UnitRanges rg;
  unit_ranges_fill(geo, u, Mu, has_list, anchor, rg);
  __syncthreads();
  int tail_lo, n_tail, anc_u;
  unit_spans(rg, Mu, &tail_lo, &n_tail, &anc_u);
  int t0, t1;
  split_range(nnode + n_tail, splits, sp, kTile, &t0, &t1);
  const int64_t row0 = (int64_t)bg_of(geo, u) * geo.Ncap;
  const bf16_t* Ku = K + row0 * D;
  const bf16_t* Vu = V + row0 * D;
  const uint32_t* nodes = l1.nodes + u * l1.stride;
  const uint32_t* masks = l1.masks + u * l1.stride;
  uint32_t* sV = smem + wave * kTile * RW;

  bf16x8_t qb[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (mem < Mu) v = ld16(Q + (int64_t)qh_of(geo, u, mem) * D + 32 * kc + 8 * grp);
    qb[kc] = as_bf16x8(v);
  }
  f32x4_t acc[KC][2];
#pragma unroll
  for (int c = 0; c < KC; ++c) acc[c][0] = acc[c][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;

  // Token ids and member masks of a tile are worked out once, one lane per row (lanes
  // 0..31), by region (uniform across the wave, so the branches are scalar): anchor tiles (0)
  // cover tokens [0, anchor) for the members that see them; list tiles (1) read the staged
  // list (entry i / b - nbase) and skip tokens below the anchor; tail tiles (2) map work
  // index i to token tail_lo + (i - nnode) for the members whose tail holds it (every
  // member without query positions). Past `lim`: token 0, no member (its loads stay in
  // bounds). They go to this wave's slot in LDS; token ids are stored row-permuted so that
  // each lane's V rows (lane / CH + RPI j) sit in adjacent words.
  int* s_tok = s_tt + wave * 2 * kTile;
  uint32_t* s_mk = s_tm + wave * 2 * kTile;
  auto prepare = [&](int region, int slot, int base, int lim, int nbase) {
    if (lane < kTile) {
      const int i = base + lane;
      int tok = 0;
      uint32_t mk = 0u;
      if (i < lim) {
        if (region == 1) {
          const int nd = (int)geo.bdiv.div((uint32_t)i);
          tok = (int)s_nodes[nd - nbase] * b + (i - nd * b);
          mk = tok < anchor ? 0u : s_masks[nd - nbase];
        } else {
          tok = region == 0 ? i : tail_lo + (i - nnode);
          // without query positions every member sees the same anchor and tail
          mk = !geo.pos ? 0xffffu
                        : (region == 0 ? anchor_members(rg, Mu, tok) : tail_members(rg, Mu, tok));
        }
      }
      s_tok[slot * kTile + (lane % RPI) * NI + lane / RPI] = tok;
      s_mk[slot * kTile + lane] = mk;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  auto issue = [&](int region, TileRegs<D>& R, int slot, int base, int lim, int nbase) {
    prepare(region, slot, base, lim, nbase);
    int tv[NI];
#pragma unroll
    for (int j = 0; j < NI; j += 4) {
      const int4 t4 = *reinterpret_cast<const int4*>(&s_tok[slot * kTile + (lane / CH) * NI + j]);
      tv[j] = t4.x;
      tv[j + 1] = t4.y;
      tv[j + 2] = t4.z;
      tv[j + 3] = t4.w;
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) R.v[j] = ld16_stream(Vu + (int64_t)tv[j] * D + 8 * (lane % CH));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 16 * h + mem;
      const int tok = s_tok[slot * kTile + (row % RPI) * NI + row / RPI];
      const bf16_t* kr = Ku + (int64_t)tok * D + 8 * grp;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) R.k[h][kc] = ld16_stream(kr + 32 * kc);
    }
  };

  auto compute = [&](const TileRegs<D>& R, int slot) {
    f32x4_t sc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sc[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        sc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(R.k[h][kc]), qb[kc], sc[h],
                                                        0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NI; ++j)
      *reinterpret_cast<uint4*>(&sV[(lane / CH + RPI * j) * RW + 4 * (lane % CH)]) = R.v[j];

    // this lane's scores: tokens base + 16h + 4 grp + r, member `mem`
    float p[8];
    float mloc = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 m4 = *reinterpret_cast<const uint4*>(&s_mk[slot * kTile + 16 * h + 4 * grp]);
      const uint32_t mrow[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = mem < Mu && ((mrow[r] >> mem) & 1u);
        const float v = ok ? sigma * sc[h][r] : -INFINITY;
        p[4 * h + r] = v;
        mloc = fmaxf(mloc, v);
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc);
    float alpha = 1.f, psum = 0.f;
    if (m_new == -INFINITY) {
#pragma unroll
      for (int v = 0; v < 8; ++v) p[v] = 0.f;
    } else {
      alpha = expf(m_run - m_new);
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        p[v] = expf(p[v] - m_new);
        psum += p[v];
      }
    }
    l_part = l_part * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      acc[c][0] *= alpha;
      acc[c][1] *= alpha;
    }
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      hi[v] = bf16_rne(p[v]);
      lo[v] = bf16_rne(p[v] - __uint_as_float(hi[v] << 16));
    }
    const bf16x8_t phi = as_bf16x8(make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16),
                                              hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16)));
    const bf16x8_t plo = as_bf16x8(make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16),
                                              lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16)));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      uint32_t dw[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int rr = (v < 4) ? 4 * grp + v : 16 + 4 * grp + (v - 4);
        dw[v] = sV[rr * RW + 16 * c + mem];
      }
      const bf16x8_t ae = as_bf16x8(make_uint4(
          (dw[0] & 0xffffu) | (dw[1] << 16), (dw[2] & 0xffffu) | (dw[3] << 16),
          (dw[4] & 0xffffu) | (dw[5] << 16), (dw[6] & 0xffffu) | (dw[7] << 16)));
      const bf16x8_t ao = as_bf16x8(make_uint4(
          (dw[0] >> 16) | (dw[1] & 0xffff0000u), (dw[2] >> 16) | (dw[3] & 0xffff0000u),
          (dw[4] >> 16) | (dw[5] & 0xffff0000u), (dw[6] >> 16) | (dw[7] & 0xffff0000u)));
      acc[c][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ae, phi, acc[c][0], 0, 0, 0);
      acc[c][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ae, plo, acc[c][0], 0, 0, 0);
      acc[c][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, phi, acc[c][1], 0, 0, 0);
      acc[c][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, plo, acc[c][1], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // wave tiles from `base` to `lim`, step kDecWaves tiles, the next tile's loads in flight
  const int step = kDecWaves * kTile;
  auto run_tiles = [&](int region, int base, int lim, int nbase) {
    if (base >= lim) return;
    TileRegs<D> A, Bq;
    issue(region, A, 0, base, lim, nbase);
    while (true) {
      const int n1 = base + step;
      issue(region, Bq, 1, n1, lim, nbase);  // past lim this reads token 0, masked out
      compute(A, 0);
      if (n1 >= lim) break;
      const int n2 = n1 + step;
      issue(region, A, 0, n2, lim, nbase);
      compute(Bq, 1);
      if (n2 >= lim) break;
      base = n2;
    }
  };

  if (sp == 0 && wave == 0) {
    for (int base = 0; base < anc_u; base += kTile) {
      TileRegs<D> R;
      issue(0, R, 0, base, anc_u, 0);
      compute(R, 0);
    }
  }

  // list tiles, in chunks of the union list small enough to stage in LDS, then the tail
  // (region 2) as one more chunk that stages nothing
  const int span = ((kNodeChunk - 1) * b) / kTile * kTile;  // tokens per chunk
  const int l_end = min(t1, nnode);
  const int a0 = max(t0, nnode);
  for (int c0 = t0; c0 < t1;) {
    const bool tail = c0 >= l_end;
    const int c1 = tail ? t1 : min(c0 + span, l_end);
    const int nbase = c0 / b;
    if (!tail) {
      const int nend = (c1 - 1) / b + 1;
      __syncthreads();
      for (int i = threadIdx.x; i < nend - nbase; i += kDecThreads) {
        s_nodes[i] = nodes[nbase + i];
        s_masks[i] = masks[nbase + i];
      }
      __syncthreads();
    }
    const int start = tail ? a0 : c0;
    run_tiles(tail ? 2 : 1, start + wave * kTile, c1, nbase);
    c0 = tail ? t1 : c1;
  }

  // per-member totals over the 4 lanes of a member, then hand the states to LDS
  l_part += __shfl_xor(l_part, 16, 64);
  l_part += __shfl_xor(l_part, 32, 64);
  __syncthreads();  // every wave is done with its V tile before the LDS is reused
  float* sm = reinterpret_cast<float*>(smem);
  float* sl = sm + kDecWaves * kMaxMembers;
  float* so = sl + kDecWaves * kMaxMembers;
  if (grp == 0) {
    sm[wave * kMaxMembers + mem] = m_run;
    sl[wave * kMaxMembers + mem] = l_part;
  }
#pragma unroll
  for (int c = 0; c < KC; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int par = 0; par < 2; ++par)
        so[(wave * kMaxMembers + mem) * D + 32 * c + 8 * grp + 2 * r + par] = acc[c][par][r];
  __syncthreads();
  write_partial<D>(u, sp, splits, Mu, sm, sl, so, part);
}

}  // namespace

hipError_t launch_decode(const Geom& geo, int dtype, const void* K, const void* V,
                         const void* Q, const LevelBufs& l1, int has_list, int anchor,
                         int splits, float* partials, hipStream_t s) {
  if (splits < 1 || splits > kMaxSplits) return hipErrorInvalidValue;
  dim3 grid(splits, geo.U);
  const float sigma = 1.0f / sqrtf((float)geo.D);
#define ZHA_DEC(KERNEL, T)                                                                    \
  hipLaunchKernelGGL(KERNEL, grid, dim3(kDecThreads), 0, s, geo, (const T*)K, (const T*)V,     \
                     (const T*)Q, l1, has_list, anchor, splits, partials,  \
                     sigma)
  if (dtype == ZHA_BF16) {
    if (geo.D == 64) ZHA_DEC((decode_mfma_kernel<64>), bf16_t);
    else ZHA_DEC((decode_mfma_kernel<128>), bf16_t);
  } else {
    if (geo.D == 64) ZHA_DEC((decode_valu_kernel<float, 64>), float);
    else ZHA_DEC((decode_valu_kernel<float, 128>), float);
  }
#undef ZHA_DEC
  return hipGetLastError();
}

hipError_t launch_combine(const Geom& geo, int splits, const float* partials, float* O,
                          hipStream_t s) {
  dim3 grid(geo.U, geo.Tb * geo.G);
  if (geo.D == 64)
    hipLaunchKernelGGL((combine_kernel<64>), grid, dim3(kCombThreads), 0, s, geo, splits,
                       partials, O);
  else
    hipLaunchKernelGGL((combine_kernel<128>), grid, dim3(kCombThreads), 0, s, geo, splits,
                       partials, O);
  return hipGetLastError();
}

}  // namespace zha
