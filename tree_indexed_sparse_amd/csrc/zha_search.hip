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
// member. Each member then selects over its own sub-frontier and records the nodes it
// keeps as bits by node id. A level's frontier is indexed by node id: entry k is node k,
// and its score launch ORs the members' bits of the parent k / b into the entry's member
// mask and scores only the rows of parents some member kept (with b a multiple of 4 each
// workgroup lists its kept parents in LDS and walks their rows, so a sparse level costs
// its kept rows, not the whole tree). Only level 1 is compacted in memory, into the
// kept-node list the decode reads and the members' token lists.
//
// A level = a score and a select launch (plus the compaction at level 1). Kernel
// boundaries order them; no kernel here uses a device-scope fence.

#include "zha_internal.h"
#include "zha_mxfp4.h"

namespace zha {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kScoreThreads = 256;
constexpr int kScoreEntries = 2048;  // most frontier entries per workgroup (512 per wave)

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kBuckets = 512;
constexpr int kCand = 2048;
constexpr float kMaxSpread = 32.0f;             // exp(-32) * 2^42 < 1: lower masses are 0

constexpr int kCompactThreads = 1024;
constexpr int kCompactChunk = 16384;            // frontier entries per compaction step

// The unit's member masks of parents p0 .. p0 + np - 1 (bit m: member m kept the parent),
// ORed from the members' kept bits one level up: into sPm and into the frontier's parent
// masks, which the level's selection and compaction read. sPw: kMaxMembers * wcap words of
// staging. Every thread calls this; it ends with a barrier.
template <int NT>
__device__ __forceinline__ void stage_parent_masks(const Geom& geo, const Frontier& fr, int u,
                                                   int Mu, int p0, int np, uint32_t* sPw,
                                                   int wcap, uint32_t* sPm) {
  const int w0 = p0 >> 5;
  const int nw = ((p0 + np - 1) >> 5) - w0 + 1;  // <= wcap
  for (int i = threadIdx.x; i < Mu * nw; i += NT) {
    const int mm = i / nw, wd = i - mm * nw;
    sPw[mm * wcap + wd] = fr.pbits[(int64_t)qh_of(geo, u, mm) * fr.pwords + w0 + wd];
  }
  __syncthreads();
  uint32_t* gm = fr.pmask + (int64_t)u * fr.pstride;
  for (int i = threadIdx.x; i < np; i += NT) {
    const int j = p0 + i, wd = (j >> 5) - w0, bt = j & 31;
    uint32_t mk = 0u;
    for (int mm = 0; mm < Mu; ++mm) mk |= ((sPw[mm * wcap + wd] >> bt) & 1u) << mm;
    sPm[i] = mk;
    gm[j] = mk;
  }
  __syncthreads();
}

// Token list run: dst[j] = nodes[j / b] * b + j % b for j < ntok, skipping tokens below
// `anc` (the anchor tokens, written separately). Threads t = 0, nt, 2 nt, ... of the nt
// taking part write the 16-byte aligned groups of four with one store each and the few
// entries before the first aligned group and after the last with 4-byte stores, so every
// store instruction covers contiguous, aligned memory however the run starts.
__device__ __forceinline__ void write_token_run(int32_t* dst, int ntok, const uint32_t* nodes,
                                                const FastDiv& bd, int anc, int t, int nt) {
  const int b = (int)bd.d;
  auto tok_of = [&](int j) {
    const int q = (int)bd.div((uint32_t)j);
    return (int)nodes[q] * b + (j - q * b);
  };
  const int head = min((int)((4u - (uint32_t)(((uintptr_t)dst >> 2) & 3u)) & 3u), ntok);
  const int groups = (ntok - head) >> 2;
  const int tail0 = head + 4 * groups;
  for (int j = t; j < head; j += nt) {
    const int tok = tok_of(j);
    if (tok >= anc) dst[j] = tok;
  }
  for (int g = t; g < groups; g += nt) {
    const int j = head + 4 * g;
    const int t0 = tok_of(j), t1 = tok_of(j + 1), t2 = tok_of(j + 2), t3 = tok_of(j + 3);
    if (t0 >= anc && t1 >= anc && t2 >= anc && t3 >= anc) {
      *reinterpret_cast<int4*>(dst + j) = make_int4(t0, t1, t2, t3);
    } else {
      if (t0 >= anc) dst[j] = t0;
      if (t1 >= anc) dst[j + 1] = t1;
      if (t2 >= anc) dst[j + 2] = t2;
      if (t3 >= anc) dst[j + 3] = t3;
    }
  }
  for (int j = tail0 + t; j < ntok; j += nt) {
    const int tok = tok_of(j);
    if (tok >= anc) dst[j] = tok;
  }
}

// ------------------------------------------------------------------------------ score
// Scores of a level's union frontier for every member of a unit: sigma * q . X per row,
// each row read once per call. The float32 router's rows are scored on the vector units
// (score_rows_kernel, below); the FP4 router's MXFP4 rows on the scaled FP4 MFMA
// (score_fp4_kernel).

// ---- FP4 router: the query and the summary rows as MXFP4 operands of
// v_mfma_scale_f32_16x16x128_f8f6f4 (both in E2M1). Lane l (row or query column l % 16,
// 32-element block l / 16) holds that block's 16 code bytes and its E8M0 scale byte; for
// d = 64 the blocks 2 and 3 are zero.
typedef int i32x8_t __attribute__((ext_vector_type(8)));

struct Fp4Rows {
  uint4 c;
  uint32_t s;
};

__device__ __forceinline__ void load_q_block(const float* qr, float (&x)[kMxBlock]) {
#pragma unroll
  for (int j = 0; j < kMxBlock / 4; ++j) {
    const float4 v = reinterpret_cast<const float4*>(qr)[j];
    x[4 * j] = v.x;
    x[4 * j + 1] = v.y;
    x[4 * j + 2] = v.z;
    x[4 * j + 3] = v.w;
  }
}
__device__ __forceinline__ void load_q_block(const bf16_t* qr, float (&x)[kMxBlock]) {
#pragma unroll
  for (int j = 0; j < kMxBlock / 8; ++j) {
    const uint4 v = reinterpret_cast<const uint4*>(qr)[j];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[8 * j + 2 * i] = __uint_as_float(w[i] << 16);
      x[8 * j + 2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

// This lane's B operand: block `blk` of the query row `qr` (or zero when !active).
template <int D, typename Tq>
__device__ __forceinline__ void fp4_query_operand(const Tq* qr, int blk, bool active,
                                                  uint4* codes, uint32_t* scale) {
  float x[kMxBlock];
  load_q_block(qr + kMxBlock * (blk % (D / kMxBlock)), x);
  uint32_t sb;
  const uint4 c = mx_encode_block(x, &sb);
  const bool on = active && blk < D / kMxBlock;
  *codes = on ? c : make_uint4(0u, 0u, 0u, 0u);
  *scale = on ? sb : 127u;
}

// This lane's A operand: block `blk` of row `node` (a valid row). Nothing is masked: for
// d = 64 the query's blocks 2 and 3 are zero, so those lanes' codes (re-read from blocks
// 0 and 1) add nothing, and rows past the frontier are scored but never stored. Selecting
// on the loaded values would make every load wait at once.
template <int D>
__device__ __forceinline__ void fp4_row_operand(const uint8_t* codes, const uint8_t* scales,
                                                uint32_t node, int blk, Fp4Rows& R) {
  constexpr int NB = D / kMxBlock;
  R.c = __builtin_bit_cast(
      uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
                 codes + (int64_t)node * (D / 2) + 16 * (blk % NB))));
  R.s = scales[(int64_t)node * NB + blk % NB];
}

// The empty asm statement consumes the product where it is computed: without it the
// compiler may sink the MFMA, and the selects that build its operands, into a branch that
// only some lanes take (the score stores), although the instruction reads every lane.
__device__ __forceinline__ f32x4_t fp4_mfma(const Fp4Rows& R, uint4 qc, uint32_t qs, f32x4_t c) {
  const i32x8_t a = {(int)R.c.x, (int)R.c.y, (int)R.c.z, (int)R.c.w, 0, 0, 0, 0};
  const i32x8_t b = {(int)qc.x, (int)qc.y, (int)qc.z, (int)qc.w, 0, 0, 0, 0};
  f32x4_t d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 0, (int)R.s, 0,
                                                               (int)qs);
  asm volatile("" : "+v"(d));
  return d;
}

// S^T[row][member] on v_mfma_scale_f32_16x16x128_f8f6f4, 16 frontier rows per MFMA block:
// lane (row or member l % 16, 32-element block l / 16) holds that block's codes and scale;
// the C block leaves four consecutive rows of one member per lane, stored as one 16-byte
// write. Each wave walks its row blocks with the next block's loads in flight while the
// current one is multiplied.
template <int D, typename Tq>
__global__ __launch_bounds__(kScoreThreads) void score_fp4_kernel(
    Geom geo, const Tq* __restrict__ Q, Frontier fr, float* __restrict__ S, int64_t S_stride,
    float sigma, int ent, float* __restrict__ pmax, float* __restrict__ pmin, int64_t pstride,
    const uint8_t* __restrict__ RC, const uint8_t* __restrict__ RS, int64_t rows_cap) {
  constexpr int kMaxParents = kScoreEntries / 2 + 2;
  constexpr int kPw = (kMaxParents + 31) / 32 + 1;
  const int kPerWave = ent / (kScoreThreads / 64);
  __shared__ uint32_t sPw[kMaxMembers * kPw];
  __shared__ uint32_t sPm[kMaxParents];
  __shared__ float sRed[2][kScoreThreads / 64][16];

  const int u = blockIdx.y;
  const bool has_parent = fr.pbits != nullptr;
  const int F = unit_entries(geo, fr, u);
  const int k_wg = blockIdx.x * ent;
  if (k_wg >= F) return;
  const int Mu = members_of(geo, u);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mem = lane & 15, grp = lane >> 4;

  const int p0 = (int)geo.bdiv.div((uint32_t)k_wg);
  // query operand: this lane's MXFP4 block of its member's query (zero past the members)
  uint4 qc = make_uint4(0u, 0u, 0u, 0u);
  uint32_t qs = 127u;
  fp4_query_operand<D, Tq>(Q + (int64_t)qh_of(geo, u, mem < Mu ? mem : 0) * D, grp, mem < Mu,
                           &qc, &qs);
  if (has_parent) {
    const int np = (int)geo.bdiv.div((uint32_t)(min(k_wg + ent, F) - 1)) - p0 + 1;
    stage_parent_masks<kScoreThreads>(geo, fr, u, Mu, p0, np, sPw, kPw, sPm);
  }
  __syncthreads();
  const uint8_t* RCu = RC + (int64_t)bg_of(geo, u) * rows_cap * (D / 2);
  const uint8_t* RSu = RS + (int64_t)bg_of(geo, u) * rows_cap * (D / kMxBlock);
  float* Srow = S + (int64_t)qh_of(geo, u, mem < Mu ? mem : 0) * S_stride;
  const int k_wave = k_wg + wave * kPerWave;
  const int nrb = k_wave < F ? min(kPerWave / 16, (F - k_wave + 15) / 16) : 0;
  float lmx = -INFINITY, lmn = INFINITY;  // over this lane's member rows
  // the entries a member's frontier can hold: below the top nodes complete for it
  const int f_mem = mem < Mu ? member_entries(geo, fr, qh_of(geo, u, mem)) : 0;

  const bool quad_parent = has_parent && geo.b % 4 == 0;
  // entries whose parent no member kept read row 0 (a cached line) and are not stored
  // for any member's selection (none has them in its frontier)
  auto load_rows = [&](Fp4Rows& R, int k) {
    const bool ok = k < F && (!has_parent || sPm[geo.bdiv.div((uint32_t)k) - p0] != 0u);
    fp4_row_operand<D>(RCu, RSu, ok ? (uint32_t)k : 0u, grp, R);
  };

  auto compute = [&](const Fp4Rows& R, int rb) {
    const f32x4_t c = fp4_mfma(R, qc, qs, f32x4_t{0.f, 0.f, 0.f, 0.f});
    // rows kb..kb+3 of member `mem`; + 0.0f turns a -0 score into +0 so float and bit
    // orders agree
    const int kb = k_wave + 16 * rb + 4 * grp;
    // with b a multiple of 4 the four rows share one parent: not stored for a member whose
    // frontier does not hold them (it never reads them)
    const bool mine = !quad_parent || ((sPm[geo.bdiv.div((uint32_t)kb) - p0] >> mem) & 1u);
    if (mem < Mu && kb < F && mine) {
      const float4 o = make_float4(sigma * c[0] + 0.0f, sigma * c[1] + 0.0f,
                                   sigma * c[2] + 0.0f, sigma * c[3] + 0.0f);
      if (kb + 3 < F) {
        *reinterpret_cast<float4*>(Srow + kb) = o;
      } else {
        Srow[kb] = o.x;
        if (kb + 1 < F) Srow[kb + 1] = o.y;
        if (kb + 2 < F) Srow[kb + 2] = o.z;
      }
      if (pmax) {
        const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int k = kb + r;
          const bool in = k < f_mem && (!has_parent ||
                                        ((sPm[geo.bdiv.div((uint32_t)k) - p0] >> mem) & 1u));
          if (in) {
            lmx = fmaxf(lmx, ov[r]);
            lmn = fminf(lmn, ov[r]);
          }
        }
      }
    }
  };

  Fp4Rows A, Bv;
  if (nrb > 0) load_rows(A, k_wave + mem);
  for (int rb = 0; rb < nrb; rb += 2) {
    if (rb + 1 < nrb) load_rows(Bv, k_wave + 16 * (rb + 1) + mem);
    compute(A, rb);
    if (rb + 1 >= nrb) break;
    if (rb + 2 < nrb) load_rows(A, k_wave + 16 * (rb + 2) + mem);
    compute(Bv, rb + 1);
  }

  if (pmax) {
    // lanes l, l^16, l^32, l^48 hold one member; then the four waves
    lmx = fmaxf(lmx, __shfl_xor(lmx, 16, 64));
    lmn = fminf(lmn, __shfl_xor(lmn, 16, 64));
    lmx = fmaxf(lmx, __shfl_xor(lmx, 32, 64));
    lmn = fminf(lmn, __shfl_xor(lmn, 32, 64));
    if (grp == 0) {
      sRed[0][wave][mem] = lmx;
      sRed[1][wave][mem] = lmn;
    }
    __syncthreads();
    if (threadIdx.x < Mu) {
      float mx = sRed[0][0][threadIdx.x], mn = sRed[1][0][threadIdx.x];
#pragma unroll
      for (int w = 1; w < kScoreThreads / 64; ++w) {
        mx = fmaxf(mx, sRed[0][w][threadIdx.x]);
        mn = fminf(mn, sRed[1][w][threadIdx.x]);
      }
      const int64_t at = (int64_t)qh_of(geo, u, threadIdx.x) * pstride + blockIdx.x;
      pmax[at] = mx;
      pmin[at] = mn;
    }
  }
}

// ---- float32 rows, coalesced: the scoring of the float32 router. A row of D floats is
// split over LPR lanes, each taking DPL = D / LPR dims as DPL / 4 16-byte loads placed
// 16 LPR bytes apart, so every load instruction reads RPI = 64 / LPR rows, each over
// 16 LPR contiguous bytes (whole cache lines). Each lane forms its dims' partial dot
// product with every member's query; a butterfly over the row's lanes then halves the
// member set at each exchange (the lane whose exchange bit is set keeps the upper half,
// its partner the lower, each adding the other's copy of the half it keeps), so after
// log2(M) exchanges a lane holds one member's sum over its lane group and the remaining
// exchanges complete it: lane sub = l % LPR ends with member sub / (LPR / M). Exchanges
// within 16 lanes are DPP moves (partners by quad permutation or by mirroring within 8 or
// 16 lanes: any pairing across the split works, since each step sums disjoint pairs).
// The four waves of a workgroup take its rows in turn, 8 at a time, so the workgroup
// reads one contiguous stream. Scores stay in LDS until the last row is loaded and then
// leave as 16-byte stores per member: a store issued while row loads are in flight would
// make the compiler wait for every outstanding load before the next use of one (it cannot
// order loads and stores on the one counter). Two groups of row loads are in flight per
// wave; rows are read once per call (non-temporal loads).
constexpr int kRowEntries = 1024;            // most frontier entries per workgroup
constexpr int kRowGroup = 8;                 // rows per load group (16: 102.8 us, 8: 99 us at level 1)

__device__ __forceinline__ void load_q4(const float* q, float* o) {
  const float4 v = *reinterpret_cast<const float4*>(q);
  o[0] = v.x;
  o[1] = v.y;
  o[2] = v.z;
  o[3] = v.w;
}
__device__ __forceinline__ void load_q4(const bf16_t* q, float* o) {
  const uint2 v = *reinterpret_cast<const uint2*>(q);
  o[0] = __uint_as_float(v.x << 16);
  o[1] = __uint_as_float(v.x & 0xffff0000u);
  o[2] = __uint_as_float(v.y << 16);
  o[3] = __uint_as_float(v.y & 0xffff0000u);
}

// the value of this lane's partner across lane bit log2(DIST)
template <int DIST>
__device__ __forceinline__ float lane_xchg(float v) {
  const int x = __float_as_int(v);
  if constexpr (DIST == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
  else if constexpr (DIST == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
  else if constexpr (DIST == 4) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false));
  else if constexpr (DIST == 8) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false));
  else return __shfl_xor(v, DIST, 64);
}

// halving exchanges over lane bits log2(DIST), log2(DIST / 2), ... while C values remain
template <int C, int DIST>
struct MemberHalve {
  static __device__ __forceinline__ void run(float* v, int lane) {
    if constexpr (C > 1) {
      const bool hi = (lane & DIST) != 0;
#pragma unroll
      for (int t = 0; t < C / 2; ++t) {
        const float send = hi ? v[t] : v[t + C / 2];
        const float keep = hi ? v[t + C / 2] : v[t];
        v[t] = keep + lane_xchg<DIST>(send);
      }
      MemberHalve<C / 2, DIST / 2>::run(v, lane);
    } else if constexpr (DIST >= 1) {
      v[0] += lane_xchg<DIST>(v[0]);
      MemberHalve<1, DIST / 2>::run(v, lane);
    }
  }
};

template <int D, typename Tq, int M, int LPR>
__global__ __launch_bounds__(kScoreThreads) void score_rows_kernel(
    Geom geo, const float* __restrict__ X, int64_t X_unit_stride, const Tq* __restrict__ Q,
    Frontier fr, float* __restrict__ S, int64_t S_stride, float sigma, int ent,
    float* __restrict__ pmax, float* __restrict__ pmin, int64_t pstride) {
  constexpr int DPL = D / LPR;                // dims per lane
  constexpr int NLD = DPL / 4;                // 16-byte loads per lane per row
  constexpr int RPI = 64 / LPR;               // rows per load instruction
  constexpr int RL = LPR / M;                 // lanes per member once reduced
  static_assert(M <= LPR && (M & (M - 1)) == 0, "M: a power of two up to the lanes of a row");
  static_assert(NLD >= 1 && NLD * 4 * LPR == D, "whole 16-byte loads per lane");
  constexpr int NW = kScoreThreads / 64;
  constexpr int IPG = kRowGroup / RPI;        // row slots per lane per load group
  constexpr int kMaxParents = kRowEntries / 2 + 2;
  constexpr int kPw = (kMaxParents + 31) / 32 + 1;
  static_assert(M % NW == 0, "members spread evenly over the waves for the stores");
  static_assert(kRowEntries / 4 <= kScoreThreads,
                "with b a multiple of 4 a workgroup's whole parents fit one per thread");
  __shared__ uint32_t sPw[kMaxMembers * kPw];
  __shared__ uint32_t sPm[kMaxParents];
  __shared__ uint16_t sKept[kMaxParents];  // the kept parents, ascending (compact mode)
  __shared__ float sS[M][kRowEntries];

  const int u = blockIdx.y;
  const bool has_parent = fr.pbits != nullptr;
  const int F = unit_entries(geo, fr, u);
  const int k_wg = blockIdx.x * ent;
  if (k_wg >= F) return;
  const int k_end = min(k_wg + ent, F);
  const int Mu = members_of(geo, u);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPR, rin = lane / LPR;
  const int p0 = (int)geo.bdiv.div((uint32_t)k_wg);
  // this lane's dims of every member's query, zero past the unit's members
  float qv[M][DPL];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const Tq* qr = Q + (int64_t)qh_of(geo, u, m < Mu ? m : 0) * D + 4 * sub;
#pragma unroll
    for (int j = 0; j < NLD; ++j) load_q4(qr + 4 * LPR * j, &qv[m][4 * j]);
  }
  // With b a multiple of 4 a member's scores are stored only over its own frontier (the
  // children of the parents it kept), so the rows of parents no member kept are never
  // needed: when the workgroup's range holds whole parents and at least an eighth of them
  // were kept by no member, only the kept parents' rows are scored (compact mode), in
  // ascending order. Otherwise every row of the range is (rows of unkept parents read row
  // 0, a cached line, and their scores are not stored). The stored scores are the same
  // either way.
  const bool quad_parent = has_parent && geo.b % 4 == 0;
  bool compact = false;
  int n_rows = k_end - k_wg;  // rows scored by the workgroup
  if (has_parent) {
    const int np = (int)geo.bdiv.div((uint32_t)(k_end - 1)) - p0 + 1;
    stage_parent_masks<kScoreThreads>(geo, fr, u, Mu, p0, np, sPw, kPw, sPm);
    if (quad_parent && k_wg % geo.b == 0 && k_end % geo.b == 0) {
      // whole parents: np = (k_end - k_wg) / b <= kRowEntries / 4 = kScoreThreads
      const int nk = __syncthreads_count((int)threadIdx.x < np && sPm[threadIdx.x] != 0u);
      // compact mode's row addressing (a division and an LDS read per row slot ahead of
      // the loads) costs about a tenth of a dense row's time: it pays once an eighth of
      // the parents or more are unkept
      if (8 * nk <= 7 * np) {
        if (wave == 0) {
          int at = 0;
          for (int base = 0; base < np; base += 64) {
            const int i = base + lane;
            const bool kept = i < np && sPm[i] != 0u;
            const uint64_t bal = __ballot(kept);
            if (kept) sKept[at + __popcll(bal & ((1ull << lane) - 1ull))] = (uint16_t)i;
            at += __popcll(bal);
          }
        }
        __syncthreads();
        compact = true;
        n_rows = nk * geo.b;
      }
    }
  }
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int e = 0; e < DPL; ++e) qv[m][e] = m < Mu ? qv[m][e] : 0.f;
  __syncthreads();
  const float* Xu = X + (int64_t)bg_of(geo, u) * X_unit_stride + 4 * sub;
  // the workgroup's rows in groups of kRowGroup, taken by the waves in turn, so the four
  // waves read one contiguous stream
  const int groups_wg = (n_rows + kRowGroup - 1) / kRowGroup;
  const int n_groups = groups_wg > wave ? (groups_wg - wave + NW - 1) / NW : 0;

  // Every group's loads are issued unconditionally (rows past the workgroup's rows read its
  // last row again, a line already in cache; in dense mode, rows whose parent no member
  // kept read row 0, and no member's selection reads their scores): a branch around a load
  // would make the compiler wait for all outstanding loads where the paths join.
  typedef f32x4_t Group[IPG][NLD];
  // sigma * q . x for every member over one row slot, left by the butterfly in the lanes
  // sub % RL == 0 (member sub / RL)
  auto row_score = [&](const f32x4_t (&xr)[NLD]) {
    float v[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float a = xr[0].x * qv[m][0];
      a = fmaf(xr[0].y, qv[m][1], a);
      a = fmaf(xr[0].z, qv[m][2], a);
      a = fmaf(xr[0].w, qv[m][3], a);
#pragma unroll
      for (int j = 1; j < NLD; ++j) {
        a = fmaf(xr[j].x, qv[m][4 * j], a);
        a = fmaf(xr[j].y, qv[m][4 * j + 1], a);
        a = fmaf(xr[j].z, qv[m][4 * j + 2], a);
        a = fmaf(xr[j].w, qv[m][4 * j + 3], a);
      }
      v[m] = a;
    }
    MemberHalve<M, LPR / 2>::run(v, lane);
    // + 0.0f turns a -0 score into +0 so float and bit orders agree
    return sigma * v[0] + 0.0f;
  };

  if (!compact) {
    // dense: every row of the range; rows whose parent no member kept read row 0
    auto load_group = [&](Group& x, int g) {
      uint32_t node[IPG];
#pragma unroll
      for (int i = 0; i < IPG; ++i) {
        const uint32_t kc =
            (uint32_t)min(k_wg + (g * NW + wave) * kRowGroup + i * RPI + rin, k_end - 1);
        const uint32_t pm = sPm[has_parent ? geo.bdiv.div(kc) - p0 : 0];
        node[i] = (!has_parent || pm != 0u) ? kc : 0u;
      }
#pragma unroll
      for (int i = 0; i < IPG; ++i)
#pragma unroll
        for (int j = 0; j < NLD; ++j)
          x[i][j] = __builtin_nontemporal_load(
              reinterpret_cast<const f32x4_t*>(Xu + (int64_t)node[i] * D + 4 * LPR * j));
    };
    auto compute_group = [&](const Group& x, int g) {
      const int r0 = (g * NW + wave) * kRowGroup;  // row of the workgroup's range
#pragma unroll
      for (int i = 0; i < IPG; ++i) {
        const float sc = row_score(x[i]);
        // slots past the range store into entries past it, which nothing reads
        if (sub % RL == 0) sS[sub / RL][r0 + i * RPI + rin] = sc;
      }
    };
    if (n_groups > 0) {
      Group xa, xb;
      load_group(xa, 0);
      for (int g = 0; g < n_groups; g += 2) {
        load_group(xb, g + 1);
        compute_group(xa, g);
        load_group(xa, g + 2);
        if (g + 1 < n_groups) compute_group(xb, g + 1);
      }
    }
  } else {
    // compact: the kept parents' rows only. dst[i]: the entry (relative to k_wg) whose
    // score slot i of the group holds, or -1 for a slot past them (its load repeats the
    // last row)
    auto load_group = [&](Group& x, int (&dst)[IPG], int g) {
      uint32_t node[IPG];
#pragma unroll
      for (int i = 0; i < IPG; ++i) {
        const int r = (g * NW + wave) * kRowGroup + i * RPI + rin;
        const int rc = min(r, n_rows - 1);
        // row rc of the kept parents' rows: child rc % b of the (rc / b)-th kept parent
        const uint32_t j = geo.bdiv.div((uint32_t)rc);
        const uint32_t kc = ((uint32_t)p0 + sKept[j]) * (uint32_t)geo.b + (uint32_t)rc -
                            j * (uint32_t)geo.b;
        node[i] = kc;
        dst[i] = r < n_rows ? (int)kc - k_wg : -1;
      }
#pragma unroll
      for (int i = 0; i < IPG; ++i)
#pragma unroll
        for (int j = 0; j < NLD; ++j)
          x[i][j] = __builtin_nontemporal_load(
              reinterpret_cast<const f32x4_t*>(Xu + (int64_t)node[i] * D + 4 * LPR * j));
    };
    auto compute_group = [&](const Group& x, const int (&dst)[IPG]) {
#pragma unroll
      for (int i = 0; i < IPG; ++i) {
        const float sc = row_score(x[i]);
        if (sub % RL == 0 && dst[i] >= 0) sS[sub / RL][dst[i]] = sc;
      }
    };
    if (n_groups > 0) {
      Group xa, xb;
      int da[IPG], db[IPG];
      load_group(xa, da, 0);
      for (int g = 0; g < n_groups; g += 2) {
        load_group(xb, db, g + 1);
        compute_group(xa, da);
        load_group(xa, da, g + 2);
        if (g + 1 < n_groups) compute_group(xb, db);
      }
    }
  }
  __syncthreads();

  // scores out, after the last row load: wave w stores members w, w + NW, ..., each as one
  // contiguous run of 16-byte stores, and reduces its max and min over the member's
  // frontier entries for the chunked selection
  const int n = k_end - k_wg;
#pragma unroll
  for (int mi = 0; mi < M / NW; ++mi) {
    const int mm = wave + NW * mi;
    if (mm >= Mu) break;
    float* dst = S + (int64_t)qh_of(geo, u, mm) * S_stride + k_wg;
    const int f_mem = member_entries(geo, fr, qh_of(geo, u, mm));
    float mx = -INFINITY, mn = INFINITY;
    for (int c = 4 * lane; c < n; c += 256) {
      const float4 o = *reinterpret_cast<const float4*>(&sS[mm][c]);
      // with b a multiple of 4 the four entries share one parent: a member whose frontier
      // does not hold them never reads their scores, so they are not stored
      if (quad_parent && !((sPm[geo.bdiv.div((uint32_t)(k_wg + c)) - p0] >> mm) & 1u)) continue;
      if (c + 3 < n) {
        *reinterpret_cast<float4*>(dst + c) = o;
      } else {
        dst[c] = o.x;
        if (c + 1 < n) dst[c + 1] = o.y;
        if (c + 2 < n) dst[c + 2] = o.z;
      }
      if (pmax) {
        const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kk = k_wg + c + r;
          const bool in = c + r < n && kk < f_mem &&
                          (!has_parent || ((sPm[geo.bdiv.div((uint32_t)kk) - p0] >> mm) & 1u));
          if (in) {
            mx = fmaxf(mx, ov[r]);
            mn = fminf(mn, ov[r]);
          }
        }
      }
    }
    if (pmax) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        mn = fminf(mn, __shfl_xor(mn, off, 64));
      }
      if (lane == 0) {
        const int64_t at = (int64_t)qh_of(geo, u, mm) * pstride + blockIdx.x;
        pmax[at] = mx;
        pmin[at] = mn;
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
// trunc(e * 2^42) for e = exp(s - max) in (0, 1], from the float's bits: e = f * 2^(E-150)
// with the 24-bit significand f, so e * 2^42 = f * 2^(E - 108) (zero for subnormal e).
__device__ __forceinline__ uint64_t mass_fixed(float s, float smax) {
  const uint32_t v = __float_as_uint(expf(s - smax));
  const int E = (int)(v >> 23);
  if (E == 0) return 0ull;
  const uint64_t f = (uint64_t)((v & 0x7fffffu) | 0x800000u);
  const int sh = E - 108;
  return sh >= 0 ? (f << sh) : (sh > -64 ? (f >> -sh) : 0ull);
}
// bucket 0 holds the highest scores; t * scale stays within [0, kBuckets] because
// t is clamped to the spread that defines the scale
template <int NB = kBuckets>
__device__ __forceinline__ int bucket_of(float s, float smax, float scale, float spread) {
  const float t = fminf(smax - s, spread);
  const int b = (int)(t * scale);
  return b < NB - 1 ? b : NB - 1;
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

// The same cut for n <= 64 candidates within one wave (no block barrier): called by one
// whole wave; tmp: 64 words; writes out[0] = the cut key, out[1] = the kept candidates.
// The caller's block barrier after it publishes out.
__device__ void wave_cut(const unsigned long long* cand, unsigned long long* tmp, int n,
                         uint64_t before, uint64_t T, float mx, unsigned long long* out) {
  const int lane = threadIdx.x & 63;
  const uint64_t kk = lane < n ? cand[lane] : 0ull;
  int at = 0;
  for (int j = 0; j < n; ++j) at += cand[j] > kk;
  if (lane < n) tmp[at] = kk;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint64_t sk = lane < n ? tmp[lane] : 0ull;
  const uint64_t mk = lane < n ? mass_fixed(float_of_ord((uint32_t)(sk >> 32)), mx) : 0ull;
  const uint64_t incl = wave_incl_scan_u64(mk, lane) + before;
  if (lane < n && incl >= T && incl - mk < T) {
    out[0] = sk;
    out[1] = (uint64_t)(lane + 1);
  }
}

// The exact cut among the n (1 <= n <= NT) candidates of a boundary bucket: distinct rank
// keys in cand[0 .. n), in any order. Each is put at its rank (key descending: score
// descending, index ascending), their masses are scanned in that order starting from
// `before` (the mass of every entry ranked above the bucket), and the first candidate at
// which the cumulative mass reaches T is the cut. Returns its key; *kept = the bucket's
// candidates ranked at or above it. Called by every thread of the block; reorders cand;
// wsum: NT / 64 words, out: two words of shared memory.
template <int NT>
__device__ uint64_t small_cut(unsigned long long* cand, int n, uint64_t before, uint64_t T,
                              float mx, unsigned long long* wsum, unsigned long long* out,
                              uint32_t* kept) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t kk = tid < n ? cand[tid] : 0ull;
  int at = 0;
  for (int j = 0; j < n; ++j) at += cand[j] > kk;
  __syncthreads();
  if (tid < n) cand[at] = kk;
  __syncthreads();
  const uint64_t sk = tid < n ? cand[tid] : 0ull;
  const uint64_t mk = tid < n ? mass_fixed(float_of_ord((uint32_t)(sk >> 32)), mx) : 0ull;
  uint64_t incl = wave_incl_scan_u64(mk, lane);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  for (int w = 0; w < wave; ++w) incl += wsum[w];
  incl += before;
  if (tid < n && incl >= T && incl - mk < T) {
    out[0] = sk;
    out[1] = (uint64_t)(tid + 1);
  }
  __syncthreads();
  *kept = (uint32_t)out[1];
  return out[0];
}

constexpr int kVec = 4;                         // frontier entries per thread per tile
constexpr int kTileE = kSelThreads * kVec;      // 2048 entries per tile
constexpr int kCache = 16384;                   // frontier entries cached in LDS (64 KB)
constexpr int kUnroll = 4;                      // tiles loaded per pass iteration

struct SelShared {
  float cache[kCache];              // member scores (NaN: not a member) when F <= kCache
  unsigned long long hm[kBuckets];  // fixed-point mass per bucket / per radix digit
  uint32_t hc[kBuckets];
  unsigned long long cand[kCand];
  uint32_t tile_nodes[kTileE];
  uint32_t tile_bits[kTileE / 32];
  float red_f[2][kSelWaves];
  uint32_t wave_sum[kSelWaves];
  unsigned long long wsum64[kSelWaves];
  unsigned long long scalar_u64[4];
  uint32_t scalar_u32[8];
};

// Block-wide exclusive prefix of per-thread counts in thread order; *total = their sum.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wave_sum,
                                                    uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  __syncthreads();
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t c = wave_sum[w];
    before += (w < wave) ? c : 0u;
    tot += c;
  }
  *total = tot;
  return before + incl - v;
}

// Four consecutive frontier entries k0..k0+3 (k0 % 4 == 0) of one member: scores and
// membership, from the LDS cache or from the member's score row in global memory.
struct Quad {
  float s[kVec];
  bool in[kVec];
};

// Four consecutive entries k0..k0+3 (k0 % 4 == 0) of member m's score row, below `end`
// Every load is unconditional, from an index clamped into the row (row 0 when end is 0),
// so the loads of several quads stay in flight together; entries at or past `end` are
// not in.
__device__ __forceinline__ Quad load_quad(const float* Sq, const uint32_t* pmask, int m,
                                          const FastDiv& bd, int k0, int end) {
  Quad q;
  const int kc = k0 < end ? k0 : max((end - 1) & ~3, 0);  // rows are padded to a multiple of 4
  const float4 v = *reinterpret_cast<const float4*>(Sq + kc);
  q.s[0] = v.x;
  q.s[1] = v.y;
  q.s[2] = v.z;
  q.s[3] = v.w;
  uint32_t pw[kVec];
#pragma unroll
  for (int i = 0; i < kVec; ++i)
    pw[i] = pmask ? pmask[bd.div((uint32_t)max(min(k0 + i, end - 1), 0))] : 0xffffffffu;
#pragma unroll
  for (int i = 0; i < kVec; ++i) q.in[i] = k0 + i < end && ((pw[i] >> m) & 1u);
  return q;
}

// load_quad when b is a multiple of 4 (the quad's entries share the parent k0 / b): the
// parent mask is loaded first and a member outside the quad's parent reads the row's first
// float4 (a cached line) instead of its scores, which the score launch did not store.
__device__ __forceinline__ Quad load_quad_b4(const float* Sq, const uint32_t* pmask, int m,
                                             const FastDiv& bd, int k0, int end) {
  Quad q;
  const int kc = k0 < end ? k0 : max((end - 1) & ~3, 0);
  const bool in = (pmask[bd.div((uint32_t)kc)] >> m) & 1u;
  const float4 v = *reinterpret_cast<const float4*>(Sq + (in ? kc : 0));
  q.s[0] = v.x;
  q.s[1] = v.y;
  q.s[2] = v.z;
  q.s[3] = v.w;
#pragma unroll
  for (int i = 0; i < kVec; ++i) q.in[i] = in && k0 + i < end;
  return q;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    Geom geo, int level, const float* __restrict__ S, int64_t S_stride, Frontier fr,
    KeepBits kb, float p, int anchor, int32_t* __restrict__ sel_idx,
    int64_t cap, int32_t* __restrict__ sel_count, int32_t* __restrict__ lvl_kept) {
  __shared__ SelShared sh;
  const int qh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int u, m;
  unit_member_of(geo, qh, &u, &m);
  const int b = geo.b;
  // the member's frontier lies below Fm (the nodes under the top nodes complete for it);
  // its kept bits are written for all F entries of the level
  const int F = fr.F;
  const int vis = head_vis(geo, qh);
  const int Fm = member_entries(geo, fr, qh);
  anchor = min(anchor, vis);
  const float* Sq = S + (int64_t)qh * S_stride;
  const uint32_t* pmask = parent_masks(fr, u);
  uint32_t* kbits = kb.bits + (int64_t)qh * kb.words;
  const bool cached = Fm <= kCache;
  if (tid == 0) {
    sh.scalar_u32[0] = 0u;
    sh.scalar_u32[1] = 0u;
    sh.scalar_u64[0] = 0ull;
    sh.scalar_u64[1] = 0ull;
    sh.scalar_u64[2] = ~0ull;
  }

  auto load_global = [&](int k0) -> Quad { return load_quad(Sq, pmask, m, geo.bdiv, k0, Fm); };
  auto get = [&](int k0) -> Quad {
    if (!cached) return load_global(k0);
    Quad q;
    if (k0 >= Fm) {
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        q.s[i] = 0.f;
        q.in[i] = false;
      }
      return q;
    }
    const float4 v = *reinterpret_cast<const float4*>(&sh.cache[k0]);
    q.s[0] = v.x;
    q.s[1] = v.y;
    q.s[2] = v.z;
    q.s[3] = v.w;
#pragma unroll
    for (int i = 0; i < kVec; ++i) q.in[i] = !isnan(q.s[i]);
    return q;
  };

  // pass 0: max, min over the member's frontier; fill the LDS cache when it fits.
  // Every pass loads kUnroll tiles before using them, to keep several loads in flight.
  float mx = -INFINITY, mn = INFINITY;
  for (int base = kVec * tid; base < Fm; base += kTileE * kUnroll) {
    Quad q[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) q[j] = load_global(base + j * kTileE);
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int k0 = base + j * kTileE;
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        if (q[j].in[i]) {
          mx = fmaxf(mx, q[j].s[i]);
          mn = fminf(mn, q[j].s[i]);
        }
      }
      if (cached && k0 < Fm)
        *reinterpret_cast<float4*>(&sh.cache[k0]) =
            make_float4(q[j].in[0] ? q[j].s[0] : NAN, q[j].in[1] ? q[j].s[1] : NAN,
                        q[j].in[2] ? q[j].s[2] : NAN, q[j].in[3] ? q[j].s[3] : NAN);
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
    __syncthreads();
    // pass 1: fixed-point mass histogram over score buckets (bucket 0 = highest scores)
    for (int base = kVec * tid; base < Fm; base += kTileE * kUnroll) {
      Quad q[kUnroll];
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) q[j] = get(base + j * kTileE);
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
#pragma unroll
        for (int i = 0; i < kVec; ++i) {
          if (q[j].in[i]) {
            const int bk = bucket_of(q[j].s[i], mx, scale, spread);
            atomicAdd(&sh.hm[bk], (unsigned long long)mass_fixed(q[j].s[i], mx));
            atomicAdd(&sh.hc[bk], 1u);
          }
        }
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
      for (int base = kVec * tid; base < Fm; base += kTileE * kUnroll) {
        Quad q[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) q[j] = get(base + j * kTileE);
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
#pragma unroll
          for (int i = 0; i < kVec; ++i) {
            if (q[j].in[i] && bucket_of(q[j].s[i], mx, scale, spread) == bstar) {
              const uint32_t slot = atomicAdd(&sh.scalar_u32[0], 1u);
              sh.cand[slot] = rank_key(q[j].s[i], (uint32_t)(base + j * kTileE + i));
            }
          }
        }
      }
      __syncthreads();
      if (nb <= 64u) {
        if (wave == 0) wave_cut(sh.cand, sh.hm, (int)nb, before, T, mx, &sh.scalar_u64[2]);
        __syncthreads();
      } else if (nb <= (uint32_t)kSelThreads) {
        uint32_t kept_b;
        small_cut<kSelThreads>(sh.cand, (int)nb, before, T, mx, sh.wsum64, &sh.scalar_u64[2],
                               &kept_b);
      } else {
      int P2 = 1;
      while (P2 < (int)nb) P2 <<= 1;
      for (int i = nb + tid; i < P2; i += kSelThreads) sh.cand[i] = 0ull;
      __syncthreads();
      for (int size = 2; size <= P2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          for (int i = tid; i < P2; i += kSelThreads) {
            const int j = i ^ stride;
            if (j > i) {
              const unsigned long long x = sh.cand[i], y = sh.cand[j];
              const bool desc = (i & size) == 0;  // descending blocks give a descending result
              if (desc ? (x < y) : (x > y)) {
                sh.cand[i] = y;
                sh.cand[j] = x;
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
      }
    } else {
      // boundary bucket too large to sort: exact MSD radix select on the 64-bit rank
      // key, restricted to the boundary bucket, 8 bits per pass
      uint64_t prefix = 0, pmask_bits = 0, need = T - before;
      for (int shift = 56; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kSelThreads) sh.hm[i] = 0ull;
        __syncthreads();
        for (int k0 = kVec * tid; k0 < Fm; k0 += kTileE) {
          const Quad q = get(k0);
#pragma unroll
          for (int i = 0; i < kVec; ++i) {
            if (!q.in[i] || bucket_of(q.s[i], mx, scale, spread) != bstar) continue;
            const uint64_t key = rank_key(q.s[i], (uint32_t)(k0 + i));
            if ((key & pmask_bits) != prefix) continue;
            atomicAdd(&sh.hm[(key >> shift) & 255u], (unsigned long long)mass_fixed(q.s[i], mx));
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
          sh.scalar_u64[3] = (uint64_t)dsel;
          sh.scalar_u64[2] = run;
        }
        __syncthreads();
        const uint64_t dsel = sh.scalar_u64[3];
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
  auto keep_of = [&](float s, bool in, int k) -> bool {
    if (!in) return false;
    if (keep_all) return true;
    return s > s_cut || (s == s_cut && (uint32_t)k <= k_cut);
  };

  // anchor overlap: kept level-1 tokens below `anchor` (they sit in the first
  // ceil(anchor / b) frontier entries: entry k is node k)
  if (level == 1 && tid == 0) {
    int dup = 0;
    const int lim = min(Fm, (anchor + b - 1) / b);
    for (int k = 0; k < lim; ++k) {
      const bool in = !pmask || ((pmask[geo.bdiv.div((uint32_t)k)] >> m) & 1u);
      if (keep_of(Sq[k], in, k) && k * b < anchor) dup += min(b, anchor - k * b);
    }
    sh.scalar_u32[2] = (uint32_t)dup;
  }
  __syncthreads();
  const int dup = (level == 1) ? (int)sh.scalar_u32[2] : 0;
  int32_t* sel = sel_idx ? sel_idx + (int64_t)qh * cap : nullptr;
  if (level == 1 && sel)
    for (int i = tid; i < anchor; i += kSelThreads) sel[i] = i;

  // emit: the member's kept flags as a bit row (one 32-bit word per 32 entries, plain
  // stores); at level 1 also the token list
  uint32_t running = 0;
  Quad qn = get(kVec * tid);  // the next tile's entries are loaded one tile ahead
  if (level != 1) {
    // kept flags only: the 8 threads of a word OR their 4-bit groups across lanes and one
    // stores it; the kept count is summed once at the end
    uint32_t mine = 0;
    for (int t0 = 0; t0 < F; t0 += kTileE) {
      const int k0 = t0 + kVec * tid;
      const Quad q = qn;
      qn = get(k0 + kTileE);
      uint32_t kept_bits = 0;
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        if (keep_of(q.s[i], q.in[i], k0 + i)) {
          kept_bits |= 1u << i;
          ++mine;
        }
      }
      uint32_t wd = kept_bits << (4 * (tid % 8));
      wd |= __shfl_xor(wd, 1, 64);
      wd |= __shfl_xor(wd, 2, 64);
      wd |= __shfl_xor(wd, 4, 64);
      if (tid % 8 == 0 && k0 < F) kbits[k0 / 32] = wd;
    }
    block_excl_scan<kSelThreads>(mine, sh.wave_sum, &running);
    if (tid == 0) lvl_kept[(int64_t)qh * (geo.L + 1) + level] = (int32_t)running;
    return;
  }
  for (int t0 = 0; t0 < F; t0 += kTileE) {
    const int k0 = t0 + kVec * tid;
    const Quad q = qn;
    qn = get(k0 + kTileE);
    uint32_t kept_bits = 0, cnt = 0;
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
      if (keep_of(q.s[i], q.in[i], k0 + i)) {
        kept_bits |= 1u << i;
        ++cnt;
      }
    }
    if (tid < kTileE / 32) sh.tile_bits[tid] = 0u;
    uint32_t tile_total;
    const uint32_t r0 = block_excl_scan<kSelThreads>(cnt, sh.wave_sum, &tile_total);
    if (kept_bits) atomicOr(&sh.tile_bits[tid / 8], kept_bits << (4 * (tid % 8)));
    if (level == 1 && sel) {
      uint32_t r = r0;
#pragma unroll
      for (int i = 0; i < kVec; ++i)
        if ((kept_bits >> i) & 1u) sh.tile_nodes[r++] = (uint32_t)(k0 + i);
    }
    __syncthreads();
    const int words = min(kTileE, F - t0 + 31) / 32;
    if (tid < words) kbits[t0 / 32 + tid] = sh.tile_bits[tid];
    if (level == 1 && sel) {
      write_token_run(sel + anchor - dup + (int64_t)running * b, (int)tile_total * b,
                      sh.tile_nodes, geo.bdiv, anchor, tid, kSelThreads);
    }
    __syncthreads();
    running += tile_total;
  }
  if (tid == 0) {
    lvl_kept[(int64_t)qh * (geo.L + 1) + level] = (int32_t)running;
    if (level == 1) sel_count[qh] = anchor + (int32_t)running * b - dup;
  }
}

// -------------------------------------------------------------- fused upper levels
// The levels whose frontier holds at most kTopFuse entries (the top levels of a deep tree)
// run in one launch instead of three per level. Each query head walks them top-down in
// its own workgroup, with its own frontier (the children of the nodes it kept one level
// up), scores and kept list in LDS; it records the nodes it keeps at each level as a
// bitmap by node id, which the next level's score launch ORs per unit into its parent
// masks.
// Per level and head:
//   score:  sigma * q . X for every frontier row; a row is split over D / 4 lanes that
//           each take four dims, and the partial sums are added across those lanes;
//   select: a fixed-point mass histogram over score buckets below the max finds the
//           bucket where the cumulative mass (scores descending) reaches ceil(p Z); one
//           wave ranks that bucket's entries (at most 64) by (score desc, index asc) and
//           scans their masses to the exact cut. A larger boundary bucket (many equal
//           scores) takes a mass-weighted radix select over the 32-bit score ordinal:
//           the entries tied at the cut share one mass, so the first ceil(rest / mass)
//           of them by index are kept. Both keep the same (score desc, index asc)
//           prefix as the other selection paths.
constexpr int kTopThreads = 1024;
constexpr int kTopWaves = kTopThreads / 64;
constexpr int kTopFuse = 1024;                   // levels of at most this many nodes are fused
// frontier entries the kernel holds: a fused level's frontier holds at most its nodes
constexpr int kTopMax = kTopFuse;
// row loads per lane per batch: 4 at kTopThreads, so a CU has the same rows in flight
// with one workgroup of kTopThreads or two of half that size (8 spilled registers and
// measured slower: 38.7 against 33.5 us for the top levels at 256K deep; 2 and 3 measured
// the same as 4)
template <int NT>
constexpr int top_unroll() { return 4 * NT / kTopThreads; }
// The kernel fits in 128 VGPRs, four waves per SIMD: one workgroup of kTopThreads per
// CU, or two of kTopThreads / 2. The smaller one runs when there are more query heads than
// CUs, so that two heads share a CU and each hides the other's barriers and load latency.
constexpr int kTopMinWaves = 4;
constexpr int kTopWords = kTopMax / 32;          // bitmap words per (head, level)

struct TopLevels {
  int64_t xoff[ZHA_MAX_LEVELS + 1];     // float offset of level l in the pyramid
  int64_t xstride[ZHA_MAX_LEVELS + 1];  // floats per (sequence, KV head) at level l
};

constexpr int kTopBuckets = 256;                 // score buckets of the selection
static_assert(kTopMax * sizeof(float) >= 64 * sizeof(unsigned long long),
              "the score array holds the boundary bucket's candidate keys");

struct HeadTopShared {
  float S[kTopMax];
  uint32_t kn[2][kTopMax];              // kept node lists (previous level / this level)
  unsigned long long hist[kTopBuckets > 256 ? kTopBuckets : 256];  // bucket / radix digit masses
  uint32_t hcnt[kTopBuckets];
  uint32_t wcnt[kTopWaves];
  uint32_t bits[kTopWords];
  float red[kTopWaves];
  float red_mn[kTopWaves];
  unsigned long long scal64[2];
  uint32_t scal32[2];
};

template <int D, int NT>
__device__ __forceinline__ void top_rows_load(f32x4_t (&x)[top_unroll<NT>()], const float* Xu,
                                              const uint32_t* kn, bool top, const FastDiv& bd,
                                              int r0, int F, int sub, int row_in) {
  constexpr int RPB = (64 / (D / 4)) * (NT / 64);  // rows per block-wide load
#pragma unroll
  for (int i = 0; i < top_unroll<NT>(); ++i) {
    const uint32_t r = (uint32_t)min(r0 + i * RPB + row_in, F - 1);
    uint32_t node = r;
    if (!top) {
      const uint32_t q = bd.div(r);
      node = kn[q] * bd.d + (r - q * bd.d);
    }
    // plain loads: the unit's other heads read mostly the same rows, from the cache
    x[i] = *reinterpret_cast<const f32x4_t*>(Xu + (int64_t)node * D + 4 * sub);
  }
}

template <int D, int NT>
__device__ __forceinline__ void top_rows_score(const f32x4_t (&x)[top_unroll<NT>()], const float (&qv)[4],
                                               float* S, float sigma, int r0, int F, int sub,
                                               int row_in) {
  constexpr int LPR = D / 4;
  constexpr int RPB = (64 / LPR) * (NT / 64);
#pragma unroll
  for (int i = 0; i < top_unroll<NT>(); ++i) {
    float v = x[i].x * qv[0];
    v = fmaf(x[i].y, qv[1], v);
    v = fmaf(x[i].z, qv[2], v);
    v = fmaf(x[i].w, qv[3], v);
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    const int r = r0 + i * RPB + row_in;
    if (sub == 0 && r < F) S[r] = sigma * v + 0.0f;
  }
}

// FP4 router: one 16-row block per MFMA, the head's quantised query in every B column,
// so the lanes of column 0 hold the block's 16 dot products (rows 4 (l / 16) + r).
constexpr int kTopFp4Batch = 4;  // row blocks per wave in flight

template <int D, int NT>
__device__ __forceinline__ void top_fp4_score(const uint8_t* RCu, const uint8_t* RSu,
                                              const uint32_t* kn, bool top, const FastDiv& bd,
                                              int F, uint4 qc, uint32_t qs, float* S,
                                              float sigma) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mem = lane & 15, grp = lane >> 4;
  const int nblk = (F + 15) / 16;
  for (int b0 = wave; b0 < nblk; b0 += (NT / 64) * kTopFp4Batch) {
    Fp4Rows R[kTopFp4Batch];
#pragma unroll
    for (int j = 0; j < kTopFp4Batch; ++j) {
      const int blk = b0 + j * (NT / 64);
      const uint32_t r = (uint32_t)min(16 * blk + mem, F - 1);
      uint32_t node = r;
      if (!top) {
        const uint32_t q = bd.div(r);
        node = kn[q] * bd.d + (r - q * bd.d);
      }
      fp4_row_operand<D>(RCu, RSu, node, grp, R[j]);
    }
#pragma unroll
    for (int j = 0; j < kTopFp4Batch; ++j) {
      const int blk = b0 + j * (NT / 64);
      const f32x4_t c = fp4_mfma(R[j], qc, qs, f32x4_t{0.f, 0.f, 0.f, 0.f});
      if (mem == 0 && blk < nblk) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int r = 16 * blk + 4 * grp + rr;
          if (r < F) S[r] = sigma * c[rr] + 0.0f;
        }
      }
    }
  }
}

template <int D, typename Tq, bool FP4, int NT>
__global__ __launch_bounds__(NT, kTopMinWaves) void head_top_kernel(
    Geom geo, const float* __restrict__ pyramid, TopLevels tl, int l_hi, int l_lo,
    const Tq* __restrict__ Q, float p, float sigma, int32_t* __restrict__ lvl_kept,
    uint32_t* __restrict__ bitmaps, RouterView rv) {
  constexpr int EPT = kTopMax / NT;       // entries per thread (consecutive)
  static_assert(EPT >= 1 && EPT * NT == kTopMax, "whole entries per thread");
  constexpr int LPR = D / 4;              // lanes per row
  constexpr int RPW = 64 / LPR;           // rows per wave-wide load
  constexpr int STEP = RPW * (NT / 64) * top_unroll<NT>();  // rows per batch
  __shared__ HeadTopShared sh;
  // workgroup b takes member b / U of unit b % U: workgroups go to the XCDs round-robin,
  // so (with U a multiple of 8) a unit's heads share one XCD's L2 for the rows they all read
  const int u = (int)blockIdx.x % geo.U, m = (int)blockIdx.x / geo.U;
  if (m >= members_of(geo, u)) return;
  const int qh = qh_of(geo, u, m);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = geo.b;
  const bool keep_all = !(p < 1.0f);
  const int sub = lane % LPR, row_in = wave * RPW + lane / LPR;
  float qv[4];
  uint4 qc = make_uint4(0u, 0u, 0u, 0u);
  uint32_t qs = 127u;
  if constexpr (FP4) {
    fp4_query_operand<D, Tq>(Q + (int64_t)qh * D, lane >> 4, true, &qc, &qs);
  } else {
    const Tq* qr = Q + (int64_t)qh * D + 4 * sub;
#pragma unroll
    for (int e = 0; e < 4; ++e) qv[e] = to_f32(qr[e]);
  }
  int cur = 0;
  // top level: every node complete for this head
  int F = head_ntop(geo, qh);
  if (F == 0) {
    // no complete top node: the head keeps nothing at any of these levels. (A non-empty
    // frontier always keeps at least one node, so below the top no frontier is empty.)
    for (int l = l_hi; l >= l_lo; --l) {
      if (tid < kTopWords) bitmaps[((int64_t)qh * (geo.L + 1) + l) * kTopWords + tid] = 0u;
      if (tid == 0) lvl_kept[(int64_t)qh * (geo.L + 1) + l] = 0;
    }
    return;
  }
  for (int l = l_hi; l >= l_lo; --l) {
    const bool top = l == l_hi;
    const float* Xu = pyramid + tl.xoff[l] + (int64_t)bg_of(geo, u) * tl.xstride[l];
    const uint32_t* kn = sh.kn[cur];
    // ---- score, two batches of rows in flight
    if constexpr (FP4) {
      const int64_t rows = tl.xstride[l] / D;
      top_fp4_score<D, NT>(rv.codes[l] + (int64_t)bg_of(geo, u) * rows * (D / 2),
                       rv.scales[l] + (int64_t)bg_of(geo, u) * rows * (D / kMxBlock), kn, top,
                       geo.bdiv, F, qc, qs, sh.S, sigma);
    } else {
      f32x4_t xa[top_unroll<NT>()], xb[top_unroll<NT>()];
      top_rows_load<D, NT>(xa, Xu, kn, top, geo.bdiv, 0, F, sub, row_in);
      for (int r0 = 0; r0 < F; r0 += 2 * STEP) {
        if (r0 + STEP < F) top_rows_load<D, NT>(xb, Xu, kn, top, geo.bdiv, r0 + STEP, F, sub, row_in);
        top_rows_score<D, NT>(xa, qv, sh.S, sigma, r0, F, sub, row_in);
        if (r0 + STEP >= F) break;
        if (r0 + 2 * STEP < F)
          top_rows_load<D, NT>(xa, Xu, kn, top, geo.bdiv, r0 + 2 * STEP, F, sub, row_in);
        top_rows_score<D, NT>(xb, qv, sh.S, sigma, r0 + STEP, F, sub, row_in);
      }
    }
    __syncthreads();

    // ---- select: thread tid takes entries k0 .. k0 + EPT - 1 (k0 = EPT tid)
    const int k0 = EPT * tid;
    float sv[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) sv[i] = sh.S[k0 + i];
    bool in[EPT];
    float mx = -INFINITY, mn = INFINITY;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      in[i] = k0 + i < F;
      if (in[i]) {
        mx = fmaxf(mx, sv[i]);
        mn = fminf(mn, sv[i]);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      mx = fmaxf(mx, __shfl_xor(mx, off, 64));
      mn = fminf(mn, __shfl_xor(mn, off, 64));
    }
    if (lane == 0) {
      sh.red[wave] = mx;
      sh.red_mn[wave] = mn;
    }
    if (tid == 0) sh.scal32[1] = 0u;  // gathered candidates
    for (int i = tid; i < kTopBuckets; i += NT) {
      sh.hist[i] = 0ull;
      sh.hcnt[i] = 0u;
    }
    __syncthreads();
    mx = sh.red[0];
    mn = sh.red_mn[0];
#pragma unroll
    for (int w = 1; w < (NT / 64); ++w) {
      mx = fmaxf(mx, sh.red[w]);
      mn = fminf(mn, sh.red_mn[w]);
    }
    uint64_t ms[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) ms[i] = in[i] ? mass_fixed(sv[i], mx) : 0ull;
    bool keep[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) keep[i] = in[i];
    if (!keep_all) {
      // Mass histogram over score buckets below the max (bucket 0 = highest scores); its
      // total is the frontier's mass Z, and the boundary bucket, where the cumulative mass
      // reaches T = ceil(p Z), is gathered and sorted by rank key (score desc, index asc)
      // when it is small, and its masses are scanned in that order to the exact cut: the
      // kept set is every entry ranked at or above it.
      const float spread = fminf(mx - mn, kMaxSpread);
      const float scale = spread > 0.f ? (float)kTopBuckets / spread : 0.f;
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        if (in[i]) {
          const int bk = bucket_of<kTopBuckets>(sv[i], mx, scale, spread);
          atomicAdd(&sh.hist[bk], (unsigned long long)ms[i]);
          atomicAdd(&sh.hcnt[bk], 1u);
        }
      }
      __syncthreads();
      if (wave == 0) {
        constexpr int per = kTopBuckets / 64;
        uint64_t loc = 0;
#pragma unroll
        for (int i = 0; i < per; ++i) loc += sh.hist[lane * per + i];
        const uint64_t incl = wave_incl_scan_u64(loc, lane);
        const uint64_t T = ceil_mul_p(p, __shfl(incl, 63, 64));
        if (lane == 0) sh.scal64[1] = T;
        const uint64_t excl = incl - loc;
        if (excl < T && incl >= T) {
          uint64_t run = excl;
          for (int i = 0; i < per; ++i) {
            const uint64_t nxt = run + sh.hist[lane * per + i];
            if (nxt >= T) {
              sh.scal32[0] = lane * per + i;  // boundary bucket
              sh.scal64[0] = run;             // mass strictly before it
              break;
            }
            run = nxt;
          }
        }
      }
      __syncthreads();
      const int bstar = (int)sh.scal32[0];
      const uint64_t before = sh.scal64[0];
      const uint64_t T = sh.scal64[1];
      const uint32_t nb = sh.hcnt[bstar];
      if (nb <= 64u) {
        // the scores were read into registers above, so the score array holds the
        // candidates now
        unsigned long long* cand = reinterpret_cast<unsigned long long*>(sh.S);
#pragma unroll
        for (int i = 0; i < EPT; ++i)
          if (in[i] && bucket_of<kTopBuckets>(sv[i], mx, scale, spread) == bstar)
            cand[atomicAdd(&sh.scal32[1], 1u)] = rank_key(sv[i], (uint32_t)(k0 + i));
        __syncthreads();
        if (wave == 0) wave_cut(cand, sh.hist, (int)nb, before, T, mx, sh.scal64);
        __syncthreads();
        const uint64_t cut = sh.scal64[0];
#pragma unroll
        for (int i = 0; i < EPT; ++i)
          keep[i] = in[i] && rank_key(sv[i], (uint32_t)(k0 + i)) >= cut;
      } else {
      // boundary bucket too large to sort: mass-weighted radix select on the score ordinal
      uint32_t ord[EPT];
#pragma unroll
      for (int i = 0; i < EPT; ++i) ord[i] = ord_of(sv[i]);
      uint64_t need = T;
      uint32_t prefix = 0u, pbits = 0u;
      for (int shift = 24; shift >= 0; shift -= 8) {
        __syncthreads();
        if (tid < 256) sh.hist[tid] = 0ull;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < EPT; ++i)
          if (in[i] && (ord[i] & pbits) == prefix)
            atomicAdd(&sh.hist[(ord[i] >> shift) & 255u], (unsigned long long)ms[i]);
        __syncthreads();
        if (wave == 0) {
          // lane l holds digits 255 - 4l .. 252 - 4l (descending); cumulative from the top
          uint64_t hv[4], loc = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            hv[i] = sh.hist[255 - 4 * lane - i];
            loc += hv[i];
          }
          const uint64_t incl = wave_incl_scan_u64(loc, lane);
          const uint64_t excl = incl - loc;
          if (excl < need && incl >= need) {  // one lane: 1 <= need <= the group's mass
            uint64_t run = excl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (run + hv[i] >= need) {
                sh.scal32[0] = 255u - 4u * lane - i;
                sh.scal64[0] = run;
                break;
              }
              run += hv[i];
            }
          }
        }
        __syncthreads();
        need -= sh.scal64[0];
        prefix |= sh.scal32[0] << shift;
        pbits |= 255u << shift;
      }
      // ties at the cut score share one mass: keep the first ceil(need / mass) by index
      const uint64_t mcut = mass_fixed(float_of_ord(prefix), mx);
      const uint64_t ties = (need + mcut - 1) / mcut;
      uint32_t ntie = 0;
#pragma unroll
      for (int i = 0; i < EPT; ++i) ntie += (in[i] && ord[i] == prefix);
      uint32_t tot;
      uint32_t rank = block_excl_scan<NT>(ntie, sh.wcnt, &tot);
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const bool tie = in[i] && ord[i] == prefix;
        keep[i] = in[i] && (ord[i] > prefix || (tie && (uint64_t)rank < ties));
        rank += tie;
      }
      }
    }
    // ---- kept list (ascending) and bitmap of kept node ids
    uint32_t nk = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) nk += keep[i];
    uint32_t kept;
    uint32_t pos = block_excl_scan<NT>(nk, sh.wcnt, &kept);
    if (tid < kTopWords) sh.bits[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      if (keep[i]) {
        uint32_t node = (uint32_t)(k0 + i);
        if (!top) {
          const uint32_t q = geo.bdiv.div(node);
          node = kn[q] * (uint32_t)b + (node - q * (uint32_t)b);
        }
        sh.kn[cur ^ 1][pos++] = node;
        atomicOr(&sh.bits[node >> 5], 1u << (node & 31));
      }
    }
    __syncthreads();
    if (tid < kTopWords)
      bitmaps[((int64_t)qh * (geo.L + 1) + l) * kTopWords + tid] = sh.bits[tid];
    if (tid == 0) lvl_kept[(int64_t)qh * (geo.L + 1) + l] = (int32_t)kept;
    cur ^= 1;
    F = (int)kept * b;
  }
}

// ------------------------------------------------------------------ chunked selection
// A large frontier runs its top-p and compaction in four launches whose workgroups each
// take one chunk of the frontier:
//   hist:  per (chunk, head): the head's max/min (from the score kernel's partials) fix
//          the bucket grid; the chunk's fixed-point masses and counts per bucket are
//          written as that chunk's histogram;
//   cut:   per head: the chunk histograms are summed, the bucket where the cumulative
//          mass reaches p is found, its entries are gathered from the score row and
//          sorted (or radix-selected) to the exact cut (score, index), and the kept
//          total is counted;
//   union: per (chunk, unit): every member's keep flags from its scores and cut, ORed
//          into per-entry member masks; kept counts per chunk, for the union and for
//          each member;
//   write: per (chunk, unit): the union list (ascending node ids and masks) at the
//          chunk's offset and, at level 1, each member's token list.
// Buckets, masses and cut are those of the single-workgroup selection, so both paths
// keep the same set.

constexpr int kWideThreads = 512;
constexpr int kWideChunk = 8192;                    // histogram chunk: 4 tiles of kTileE
constexpr int kWideTiles = kWideChunk / kTileE;
constexpr int kWB = 1024;                           // buckets of the chunked histogram
constexpr int kCutThreads = 1024;                   // one bucket per thread
constexpr int kCutWaves = kCutThreads / 64;
// Four waves per SIMD (up to 128 VGPRs): one workgroup of kCutThreads per CU, or two of
// half that size, which run when the heads outnumber the CUs.
constexpr int kCutMinWaves = 4;
constexpr int kUnionThreads = 256;
constexpr int kUnionChunk = 2048;                   // union/write chunk: 8 entries per thread
constexpr int64_t kWideMin = 16384;                 // frontiers of this size or more
static_assert(kWB <= kCutThreads || kWB % kCutThreads == 0,
              "the cut kernel gives each thread one bucket, or a whole number of them");
static_assert(kWideChunk % kTileE == 0, "histogram chunks hold whole tiles");
static_assert(kUnionChunk == 8 * kUnionThreads, "union threads take two float4 per row");

// The head's max and min member score over a frontier of F entries, from the score
// kernel's per-workgroup partials (block-wide, every thread gets both).
template <int NT>
__device__ __forceinline__ void partial_minmax(const WideSel& w, int qh, int F, float* red,
                                               float* omx, float* omn) {
  constexpr int NW = NT / 64;
  const int np = (F + w.pent - 1) / w.pent;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float mx = -INFINITY, mn = INFINITY;
  for (int i = threadIdx.x; i < np; i += NT) {
    mx = fmaxf(mx, w.pmax[(int64_t)qh * w.pstride + i]);
    mn = fminf(mn, w.pmin[(int64_t)qh * w.pstride + i]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    mn = fminf(mn, __shfl_xor(mn, off, 64));
  }
  if (lane == 0) {
    red[wave] = mx;
    red[NW + wave] = mn;
  }
  __syncthreads();
  mx = red[0];
  mn = red[NW];
#pragma unroll
  for (int v = 1; v < NW; ++v) {
    mx = fmaxf(mx, red[v]);
    mn = fminf(mn, red[NW + v]);
  }
  *omx = mx;
  *omn = mn;
}

__global__ __launch_bounds__(kWideThreads) void wide_hist_kernel(
    Geom geo, const float* __restrict__ S, int64_t S_stride, Frontier fr, WideSel w) {
  __shared__ unsigned long long hm[kWB];
  __shared__ uint32_t hc[kWB];
  __shared__ float red[2 * (kWideThreads / 64)];
  const int qh = blockIdx.y, chunk = blockIdx.x;
  int u, m;
  unit_member_of(geo, qh, &u, &m);
  const int F = unit_entries(geo, fr, u);
  const int c0 = chunk * kWideChunk;
  if (c0 >= F) return;
  const int tid = threadIdx.x;
  const float* Sq = S + (int64_t)qh * S_stride;
  const uint32_t* pmask = parent_masks(fr, u);
  const int Fm = member_entries(geo, fr, qh);  // the member's frontier lies below Fm
  const int end = min(Fm, c0 + kWideChunk);
  Quad q[kWideTiles];
  if (pmask && geo.b % 4 == 0) {
#pragma unroll
    for (int j = 0; j < kWideTiles; ++j)
      q[j] = load_quad_b4(Sq, pmask, m, geo.bdiv, c0 + j * kTileE + kVec * tid, end);
  } else {
#pragma unroll
    for (int j = 0; j < kWideTiles; ++j)
      q[j] = load_quad(Sq, pmask, m, geo.bdiv, c0 + j * kTileE + kVec * tid, end);
  }
  for (int i = tid; i < kWB; i += kWideThreads) {
    hm[i] = 0ull;
    hc[i] = 0u;
  }
  float mx, mn;
  partial_minmax<kWideThreads>(w, qh, F, red, &mx, &mn);  // its barrier orders the zeroing
  const float spread = fminf(mx - mn, kMaxSpread);
  const float scale = spread > 0.f ? (float)kWB / spread : 0.f;
#pragma unroll
  for (int j = 0; j < kWideTiles; ++j) {
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
      if (q[j].in[i]) {
        const int bk = bucket_of<kWB>(q[j].s[i], mx, scale, spread);
        atomicAdd(&hm[bk], (unsigned long long)mass_fixed(q[j].s[i], mx));
        atomicAdd(&hc[bk], 1u);
      }
    }
  }
  __syncthreads();
  const int64_t base = ((int64_t)qh * w.nch + chunk) * kWB;
  for (int i = tid; i < kWB; i += kWideThreads) {
    w.hm[base + i] = hm[i];
    w.hc[base + i] = hc[i];
  }
}

struct CutShared {
  unsigned long long cand[kCand];
  unsigned long long radix[256];
  unsigned long long wsum[kCutWaves];
  uint32_t redu[4][kCutWaves];
  float red[2 * kCutWaves];
  unsigned long long scalar_u64[4];
  uint32_t scalar_u32[4];
};

// block-wide inclusive scan of one u64 per thread; *total = the sum over the block
template <int NT>
__device__ __forceinline__ uint64_t cut_block_scan(uint64_t v, unsigned long long* wsum,
                                                   uint64_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t incl = wave_incl_scan_u64(v, lane);
  __syncthreads();
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint64_t before = 0, tot = 0;
#pragma unroll
  for (int v2 = 0; v2 < NT / 64; ++v2) {
    const uint64_t c = wsum[v2];
    before += (v2 < wave) ? c : 0ull;
    tot += c;
  }
  *total = tot;
  return before + incl;
}

template <int NT>
__global__ __launch_bounds__(NT, kCutMinWaves) void wide_cut_kernel(
    Geom geo, int level, const float* __restrict__ S, int64_t S_stride, Frontier fr,
    KeepBits kb, float p, int anchor, int32_t* __restrict__ sel_idx, int64_t cap,
    int32_t* __restrict__ sel_count, int32_t* __restrict__ lvl_kept, WideSel w) {
  __shared__ CutShared sh;
  const int qh = blockIdx.x;
  // buckets per thread: thread t owns BPT t .. BPT t + BPT - 1 (threads past kWB / BPT own
  // none)
  constexpr int BPT = kWB >= NT ? kWB / NT : 1;
  static_assert(BPT * NT >= kWB && kWB % BPT == 0, "whole buckets per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool owner = BPT * tid < kWB;
  int u, m;
  unit_member_of(geo, qh, &u, &m);
  const int b = geo.b;
  // the unit's frontier lies below F, the member's below Fm; its kept bits are written for
  // all fr.F entries of the level
  const int F = unit_entries(geo, fr, u);
  const int nch = (F + kWideChunk - 1) / kWideChunk;
  const float* Sq = S + (int64_t)qh * S_stride;
  const uint32_t* pmask = parent_masks(fr, u);
  const int vis = head_vis(geo, qh);
  const int Fm = member_entries(geo, fr, qh);
  anchor = min(anchor, vis);
  uint32_t* krow = kb.bits ? kb.bits + (int64_t)qh * kb.words : nullptr;
  const int kwords = (fr.F + 31) / 32;
  // a member with no entry at this level (it kept nothing above: no complete top node)
  // selects nothing; no entry scores above an infinite cut. Called block-uniformly.
  auto empty_result = [&]() {
    if (krow)
      for (int i = tid; i < kwords; i += NT) krow[i] = 0u;
    if (tid == 0) {
      uint32_t* rec = w.cut + 4 * (int64_t)qh;
      rec[0] = __float_as_uint(INFINITY);
      rec[1] = 0u;
      rec[2] = (uint32_t)anchor;
      rec[3] = 0u;
      lvl_kept[(int64_t)qh * (geo.L + 1) + level] = 0;
      if (level == 1) sel_count[qh] = anchor;
    }
    if (level == 1 && sel_idx)
      for (int i = tid; i < anchor; i += NT) sel_idx[(int64_t)qh * cap + i] = i;
  };
  if (Fm == 0) {
    empty_result();
    return;
  }

  // bucket totals over the chunks (thread `tid` owns buckets BPT tid .. BPT tid + BPT - 1);
  // loads issued first
  uint64_t hb[BPT];
  uint32_t cb[BPT];
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    hb[j] = 0ull;
    cb[j] = 0u;
  }
  const int64_t hbase = (int64_t)qh * w.nch * kWB + BPT * (owner ? tid : 0);
  {
    int c = 0;
    for (; c + 4 <= nch; c += 4) {
      uint64_t h[4][BPT];
      uint32_t n[4][BPT];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
          h[i][j] = w.hm[hbase + (int64_t)(c + i) * kWB + j];
          n[i][j] = w.hc[hbase + (int64_t)(c + i) * kWB + j];
        }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
          hb[j] += h[i][j];
          cb[j] += n[i][j];
        }
    }
    for (; c < nch; ++c)
#pragma unroll
      for (int j = 0; j < BPT; ++j) {
        hb[j] += w.hm[hbase + (int64_t)c * kWB + j];
        cb[j] += w.hc[hbase + (int64_t)c * kWB + j];
      }
  }
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    hb[j] = owner ? hb[j] : 0ull;
    cb[j] = owner ? cb[j] : 0u;
  }
  uint64_t hsum = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) hsum += hb[j];
  if (tid == 0) {
    sh.scalar_u32[0] = 0u;  // boundary bucket
    sh.scalar_u32[1] = 0u;  // its entry count
    sh.scalar_u32[2] = 0u;  // gathered candidates
    sh.scalar_u32[3] = 0u;  // kept candidates of the boundary bucket
    sh.scalar_u64[0] = 0ull;
    sh.scalar_u64[2] = ~0ull;
  }
  float mx, mn;
  partial_minmax<NT>(w, qh, F, sh.red, &mx, &mn);
  const float spread = fminf(mx - mn, kMaxSpread);
  const float scale = spread > 0.f ? (float)kWB / spread : 0.f;
  const bool keep_all = !(p < 1.0f);

  uint64_t Z;
  const uint64_t incl = cut_block_scan<NT>(hsum, sh.wsum, &Z);
  if (Z == 0) {  // no member entry (the top entry alone carries mass 2^42)
    empty_result();
    return;
  }
  const uint64_t T = keep_all ? Z : ceil_mul_p(p, Z);
  const uint64_t excl = incl - hsum;
  if (!keep_all && excl < T && incl >= T) {
    // exactly one of this thread's buckets has run < T <= run + its mass
    uint64_t run = excl;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      if (run < T && run + hb[j] >= T) {
        sh.scalar_u32[0] = (uint32_t)(BPT * tid + j);
        sh.scalar_u32[1] = cb[j];
        sh.scalar_u64[0] = run;
      }
      run += hb[j];
    }
  }
  __syncthreads();
  const int bstar = keep_all ? kWB : (int)sh.scalar_u32[0];
  const uint64_t before = sh.scalar_u64[0];
  const uint32_t nb = keep_all ? 0u : sh.scalar_u32[1];

  uint64_t key = ~0ull;  // keep_all: every member entry ranks at or above the cut
  if (!keep_all) {
    if (nb <= (uint32_t)kCand) {
      for (int base = kVec * tid; base < F; base += kVec * NT * kUnroll) {
        Quad q[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j)
          q[j] = load_quad(Sq, pmask, m, geo.bdiv, base + j * kVec * NT, Fm);
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
#pragma unroll
          for (int i = 0; i < kVec; ++i) {
            if (q[j].in[i] && bucket_of<kWB>(q[j].s[i], mx, scale, spread) == bstar) {
              const uint32_t slot = atomicAdd(&sh.scalar_u32[2], 1u);
              if (slot < (uint32_t)kCand)
                sh.cand[slot] = rank_key(q[j].s[i], (uint32_t)(base + j * kVec * NT + i));
            }
          }
        }
      }
      __syncthreads();
      if (nb <= 64u) {
        if (wave == 0) wave_cut(sh.cand, sh.radix, (int)nb, before, T, mx, &sh.scalar_u64[2]);
        __syncthreads();
        key = sh.scalar_u64[2];
        if (tid == 0) sh.scalar_u32[3] = (uint32_t)sh.scalar_u64[3];  // kept of the bucket
        __syncthreads();
      } else if (nb <= (uint32_t)NT) {
        uint32_t kept_b;
        key = small_cut<NT>(sh.cand, (int)nb, before, T, mx, sh.wsum, &sh.scalar_u64[2],
                                     &kept_b);
        if (tid == 0) sh.scalar_u32[3] = kept_b;  // kept entries of the boundary bucket
        __syncthreads();
      } else {
      // the exact cut among the gathered candidates: a mass-weighted radix select on the
      // score ordinal (4 passes of 8 bits) finds the cut score; the candidates tied at it
      // share one mass, and the first ceil(rest / mass) of them by index are kept
      constexpr int per = kCand / NT;
      uint32_t cord[per], cidx[per];
      uint64_t cm[per];
      bool cv[per];
#pragma unroll
      for (int i = 0; i < per; ++i) {
        const int idx = per * tid + i;
        cv[i] = idx < (int)nb;
        const uint64_t kk = cv[i] ? sh.cand[idx] : 0ull;
        cord[i] = (uint32_t)(kk >> 32);
        cidx[i] = 0xffffffffu - (uint32_t)kk;
        cm[i] = cv[i] ? mass_fixed(float_of_ord(cord[i]), mx) : 0ull;
      }
      uint64_t need = T - before;  // 1 <= need <= the boundary bucket's mass
      uint32_t prefix = 0u, pbits = 0u;
      for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) sh.radix[tid] = 0ull;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < per; ++i)
          if (cv[i] && (cord[i] & pbits) == prefix)
            atomicAdd(&sh.radix[(cord[i] >> shift) & 255u], (unsigned long long)cm[i]);
        __syncthreads();
        if (wave == 0) {
          // lane l holds digits 255 - 4l .. 252 - 4l (descending); cumulative from the top
          uint64_t hv[4], loc = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            hv[i] = sh.radix[255 - 4 * lane - i];
            loc += hv[i];
          }
          const uint64_t incl = wave_incl_scan_u64(loc, lane);
          const uint64_t excl = incl - loc;
          if (excl < need && incl >= need) {
            uint64_t run = excl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (run + hv[i] >= need) {
                sh.scalar_u32[0] = 255u - 4u * lane - i;
                sh.scalar_u64[1] = run;
                break;
              }
              run += hv[i];
            }
          }
        }
        __syncthreads();
        need -= sh.scalar_u64[1];
        prefix |= sh.scalar_u32[0] << shift;
        pbits |= 255u << shift;
      }
      const uint64_t mcut = mass_fixed(float_of_ord(prefix), mx);
      const uint64_t ties = (need + mcut - 1) / mcut;
      // candidates above the cut score, and the tied ones' count / lowest / highest index
      uint32_t nabove = 0, ntie = 0, imin = 0xffffffffu, imax = 0u;
#pragma unroll
      for (int i = 0; i < per; ++i) {
        nabove += cv[i] && cord[i] > prefix;
        if (cv[i] && cord[i] == prefix) {
          ++ntie;
          imin = min(imin, cidx[i]);
          imax = max(imax, cidx[i]);
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        nabove += __shfl_xor(nabove, off, 64);
        ntie += __shfl_xor(ntie, off, 64);
        imin = min(imin, (uint32_t)__shfl_xor(imin, off, 64));
        imax = max(imax, (uint32_t)__shfl_xor(imax, off, 64));
      }
      if (lane == 0) {
        sh.redu[0][wave] = nabove;
        sh.redu[1][wave] = ntie;
        sh.redu[2][wave] = imin;
        sh.redu[3][wave] = imax;
      }
      __syncthreads();
      nabove = ntie = imax = 0u;
      imin = 0xffffffffu;
#pragma unroll
      for (int v = 0; v < (NT / 64); ++v) {
        nabove += sh.redu[0][v];
        ntie += sh.redu[1][v];
        imin = min(imin, sh.redu[2][v]);
        imax = max(imax, sh.redu[3][v]);
      }
      uint32_t kc;
      if (ties <= 1) {
        kc = imin;
      } else if (ties >= ntie) {
        kc = imax;
      } else {
        // the ties-th lowest index among the tied candidates: count radix, low digits first
        uint32_t ip = 0u, ib = 0u, rest = (uint32_t)ties;
        for (int shift = 24; shift >= 0; shift -= 8) {
          __syncthreads();
          if (tid < 256) sh.radix[tid] = 0ull;
          __syncthreads();
#pragma unroll
          for (int i = 0; i < per; ++i)
            if (cv[i] && cord[i] == prefix && (cidx[i] & ib) == ip)
              atomicAdd(&sh.radix[(cidx[i] >> shift) & 255u], 1ull);
          __syncthreads();
          if (wave == 0) {
            // lane l holds digits 4l .. 4l + 3 (ascending)
            uint64_t hv[4], loc = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              hv[i] = sh.radix[4 * lane + i];
              loc += hv[i];
            }
            const uint64_t incl = wave_incl_scan_u64(loc, lane);
            const uint64_t excl = incl - loc;
            if (excl < rest && incl >= rest) {
              uint64_t run = excl;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                if (run + hv[i] >= rest) {
                  sh.scalar_u32[0] = 4u * lane + i;
                  sh.scalar_u64[1] = run;
                  break;
                }
                run += hv[i];
              }
            }
          }
          __syncthreads();
          rest -= (uint32_t)sh.scalar_u64[1];
          ip |= sh.scalar_u32[0] << shift;
          ib |= 255u << shift;
        }
        kc = ip;
      }
      if (tid == 0) sh.scalar_u32[3] = nabove + (uint32_t)ties;
      __syncthreads();
      key = ((uint64_t)prefix << 32) | (uint64_t)(0xffffffffu - kc);
      }
    } else {
      // boundary bucket too large to sort: exact MSD radix select on the rank key,
      // restricted to the boundary bucket, 8 bits per pass
      uint64_t prefix = 0, pbits = 0, need = T - before;
      for (int shift = 56; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += NT) sh.radix[i] = 0ull;
        __syncthreads();
        for (int k0 = kVec * tid; k0 < F; k0 += kVec * NT) {
          const Quad q = load_quad(Sq, pmask, m, geo.bdiv, k0, Fm);
#pragma unroll
          for (int i = 0; i < kVec; ++i) {
            if (!q.in[i] || bucket_of<kWB>(q.s[i], mx, scale, spread) != bstar) continue;
            const uint64_t kk = rank_key(q.s[i], (uint32_t)(k0 + i));
            if ((kk & pbits) != prefix) continue;
            atomicAdd(&sh.radix[(kk >> shift) & 255u], (unsigned long long)mass_fixed(q.s[i], mx));
          }
        }
        __syncthreads();
        if (tid == 0) {
          uint64_t r = 0;
          int dsel = 0;
          for (int dg = 255; dg >= 0; --dg) {
            if (r + sh.radix[dg] >= need) {
              dsel = dg;
              break;
            }
            r += sh.radix[dg];
          }
          sh.scalar_u64[3] = (uint64_t)dsel;
          sh.scalar_u64[1] = r;
        }
        __syncthreads();
        need -= sh.scalar_u64[1];
        prefix |= sh.scalar_u64[3] << shift;
        pbits |= 255ull << shift;
        __syncthreads();
      }
      key = prefix;
      uint32_t nk = 0;
      for (int k0 = kVec * tid; k0 < F; k0 += kVec * NT) {
        const Quad q = load_quad(Sq, pmask, m, geo.bdiv, k0, Fm);
#pragma unroll
        for (int i = 0; i < kVec; ++i)
          nk += (q.in[i] && bucket_of<kWB>(q.s[i], mx, scale, spread) == bstar &&
                 rank_key(q.s[i], (uint32_t)(k0 + i)) >= key);
      }
      if (nk) atomicAdd(&sh.scalar_u32[3], nk);
    }
  }
  const float s_cut = keep_all ? -INFINITY : float_of_ord((uint32_t)(key >> 32));
  const uint32_t k_cut = keep_all ? 0xffffffffu : 0xffffffffu - (uint32_t)key;
  // kept total: the buckets above the boundary plus the boundary's kept entries
  uint64_t kept64;
  uint64_t above = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) above += (BPT * tid + j < bstar) ? (uint64_t)cb[j] : 0ull;
  cut_block_scan<NT>(above, sh.wsum, &kept64);
  __syncthreads();
  const uint32_t kept = (uint32_t)kept64 + sh.scalar_u32[3];
  // the member's kept flags by node id, for the score launch of the level below: one entry
  // per lane, a wave's 64 flags by ballot, four entries per thread in flight (loads from
  // indices clamped below Fm; entries at or past Fm are not in)
  if (krow) {
    const int ntot = kwords * 32;
    for (int base = 0; base < ntot; base += 4 * NT) {
      float sv[4];
      uint32_t pw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kc = min(base + j * NT + tid, Fm - 1);
        sv[j] = Sq[kc];
        pw[j] = pmask ? pmask[geo.bdiv.div((uint32_t)kc)] : 0xffffffffu;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = base + j * NT + tid;
        const bool keep = k < Fm && ((pw[j] >> m) & 1u) &&
                          (sv[j] > s_cut || (sv[j] == s_cut && (uint32_t)k <= k_cut));
        const uint64_t bal = __ballot(keep);
        const int w0 = (base + j * NT + 64 * wave) >> 5;
        if (lane < 2 && w0 + lane < kwords) krow[w0 + lane] = (uint32_t)(bal >> (32 * lane));
      }
    }
  }
  if (tid == 0) {
    // anchor overlap at level 1: kept tokens below `anchor` (in the first ceil(anchor / b)
    // entries: entry k is node k)
    int dup = 0;
    if (level == 1) {
      const int lim = min(Fm, (anchor + b - 1) / b);
      for (int k = 0; k < lim; ++k) {
        const bool in = !pmask || ((pmask[geo.bdiv.div((uint32_t)k)] >> m) & 1u);
        const float sk = Sq[k];
        if (in && (sk > s_cut || (sk == s_cut && (uint32_t)k <= k_cut)) && k * b < anchor)
          dup += min(b, anchor - k * b);
      }
    }
    uint32_t* rec = w.cut + 4 * (int64_t)qh;
    rec[0] = __float_as_uint(s_cut);
    rec[1] = k_cut;
    rec[2] = (uint32_t)(anchor - dup);
    rec[3] = kept;
    lvl_kept[(int64_t)qh * (geo.L + 1) + level] = (int32_t)kept;
    if (level == 1) sel_count[qh] = anchor + (int32_t)kept * b - dup;
  }
  if (level == 1 && sel_idx)
    for (int i = tid; i < anchor; i += NT) sel_idx[(int64_t)qh * cap + i] = i;
}

// union: per (chunk of kUnionChunk entries, unit). Thread t takes entries 4t..4t+3 and
// 1024+4t..1024+4t+3 of the chunk, so each member's row is read as two coalesced float4.
__global__ __launch_bounds__(kUnionThreads) void wide_union_kernel(
    Geom geo, const float* __restrict__ S, int64_t S_stride, Frontier fr, WideSel w) {
  __shared__ float s_cut[kMaxMembers];
  __shared__ uint32_t k_cut[kMaxMembers];
  __shared__ int s_lim[kMaxMembers];
  __shared__ uint32_t cnt[kUnionThreads / 64][kMaxMembers + 1];
  const int u = blockIdx.y, chunk = blockIdx.x;
  const int F = unit_entries(geo, fr, u);
  const int c0 = chunk * kUnionChunk;
  if (c0 >= F) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Mu = members_of(geo, u);
  if (tid < Mu) {
    const int qh = qh_of(geo, u, tid);
    const uint32_t* rec = w.cut + 4 * (int64_t)qh;
    s_cut[tid] = __uint_as_float(rec[0]);
    k_cut[tid] = rec[1];
    s_lim[tid] = member_entries(geo, fr, qh);  // the member's frontier lies below this
  }
  int kk[8];
  uint32_t pm[8];
  const uint32_t* pmask = parent_masks(fr, u);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    kk[i] = c0 + (i >> 2) * (kUnionChunk / 2) + 4 * tid + (i & 3);
    pm[i] = (kk[i] < F && pmask) ? pmask[geo.bdiv.div((uint32_t)kk[i])] : 0u;
  }
  __syncthreads();
  if (!pmask) {  // top level: the members for whom the entry is a complete top node
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t msk = 0u;
      for (int mm = 0; mm < Mu; ++mm) msk |= (uint32_t)(kk[i] < s_lim[mm]) << mm;
      pm[i] = msk;
    }
  }
  uint32_t um[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  // members in groups of four, all eight row loads of a group issued together; rows are
  // padded to a multiple of 4 and chunks start at multiples of 4, so a float4 that starts
  // below F stays inside the row (past F the row's first float4 is read and ignored)
  const int off_a = kk[0] < F ? c0 + 4 * tid : 0;
  const int off_c = kk[4] < F ? c0 + kUnionChunk / 2 + 4 * tid : 0;
  // with b a multiple of 4 each float4 is one parent's entries: a member outside it reads
  // the row's first float4 (a cached line) instead of scores the score launch did not store
  const bool quad_parent = pmask && geo.b % 4 == 0;
  for (int g0 = 0; g0 < Mu; g0 += 4) {
    float4 a[4], c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int mm = min(g0 + j, Mu - 1);
      const float* Sq = S + (int64_t)qh_of(geo, u, mm) * S_stride;
      const bool ia = !quad_parent || ((pm[0] >> mm) & 1u);
      const bool ic = !quad_parent || ((pm[4] >> mm) & 1u);
      a[j] = *reinterpret_cast<const float4*>(Sq + (ia ? off_a : 0));
      c[j] = *reinterpret_cast<const float4*>(Sq + (ic ? off_c : 0));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int mm = g0 + j;
      if (mm >= Mu) break;
      const float sv[8] = {a[j].x, a[j].y, a[j].z, a[j].w, c[j].x, c[j].y, c[j].z, c[j].w};
      const float sc = s_cut[mm];
      const uint32_t kc = k_cut[mm];
      uint32_t n = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool keep = ((pm[i] >> mm) & 1u) &&
                          (sv[i] > sc || (sv[i] == sc && (uint32_t)kk[i] <= kc));
        um[i] |= (uint32_t)keep << mm;
        n += keep;
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) n += __shfl_xor(n, off, 64);
      if (lane == 0) cnt[wave][mm] = n;
    }
  }
  uint32_t nz = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) nz += um[i] != 0u;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) nz += __shfl_xor(nz, off, 64);
  if (lane == 0) cnt[wave][kMaxMembers] = nz;
  uint32_t* umg = w.umask + (int64_t)u * w.ustride + c0 + 4 * tid;
  *reinterpret_cast<uint4*>(umg) = make_uint4(um[0], um[1], um[2], um[3]);
  *reinterpret_cast<uint4*>(umg + kUnionChunk / 2) = make_uint4(um[4], um[5], um[6], um[7]);
  __syncthreads();
  if (tid <= kMaxMembers && (tid < Mu || tid == kMaxMembers)) {
    uint32_t tot = 0;
#pragma unroll
    for (int v = 0; v < kUnionThreads / 64; ++v) tot += cnt[v][tid];
    if (tid == kMaxMembers) w.ucnt[(int64_t)u * w.nuc + chunk] = tot;
    else w.mcnt[(int64_t)qh_of(geo, u, tid) * w.nuc + chunk] = tot;
  }
}

// sum of cnt[0 .. n) across one wave (every lane gets it)
__device__ __forceinline__ uint32_t wave_prefix_total(const uint32_t* cnt, int n, int lane) {
  uint32_t acc = 0;
  for (int c = lane; c < n; c += 64) acc += cnt[c];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  return acc;
}

// write (level 1): per (chunk, unit, member group). The chunk's masks are staged in LDS;
// in group 0 each wave compacts a quarter of the chunk with ballots into the union list;
// group z's wave w writes the token lists of members w + 4 z, w + 4 (z + groups), ...
// (the groups share the members' list writing).
__global__ __launch_bounds__(kUnionThreads) void wide_write_kernel(
    Geom geo, Frontier fr, LevelBufs cur, int anchor, int32_t* __restrict__ sel_idx,
    int64_t cap, WideSel w) {
  constexpr int NW = kUnionThreads / 64;
  constexpr int kPerWave = kUnionChunk / NW;
  __shared__ uint32_t s_um[kUnionChunk];
  __shared__ uint32_t wtot[NW];
  __shared__ uint32_t s_stage[NW][8 * 64];  // a wave's kept nodes of 8 x 64 entries
  const int u = blockIdx.y, chunk = blockIdx.x;
  const int b = geo.b;
  const int F = unit_entries(geo, fr, u);
  const int c0 = chunk * kUnionChunk;  // entry c0 + e is node c0 + e
  if (c0 >= F) {
    // a unit whose queries see no complete top node has an empty list
    if (F == 0 && chunk == 0 && blockIdx.z == 0 && threadIdx.x == 0) cur.count[u] = 0u;
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Mu = members_of(geo, u);
  const int nchunks = (F + kUnionChunk - 1) / kUnionChunk;
  {
    const uint32_t* umg = w.umask + (int64_t)u * w.ustride + c0;
    const uint4 a = *reinterpret_cast<const uint4*>(umg + 4 * tid);
    const uint4 c = *reinterpret_cast<const uint4*>(umg + kUnionChunk / 2 + 4 * tid);
    *reinterpret_cast<uint4*>(&s_um[4 * tid]) = a;
    *reinterpret_cast<uint4*>(&s_um[kUnionChunk / 2 + 4 * tid]) = c;
  }
  const uint32_t before = wave_prefix_total(w.ucnt + (int64_t)u * w.nuc, chunk, lane);
  __syncthreads();
  // entries past F hold zero masks (the union kernel wrote them so)
  const int e0 = wave * kPerWave;
  uint32_t mine = 0;
  for (int r = 0; r < kPerWave / 64; ++r)
    mine += __popcll(__ballot(s_um[e0 + 64 * r + lane] != 0u));
  if (lane == 0) wtot[wave] = mine;
  __syncthreads();
  uint32_t pos = before;
  for (int v = 0; v < wave; ++v) pos += wtot[v];
  uint32_t* onodes = cur.nodes + u * cur.stride;
  uint32_t* omasks = cur.masks + u * cur.stride;
  const int zg = blockIdx.z, ng = gridDim.z;
  if (zg == 0) {
    for (int r = 0; r < kPerWave / 64; ++r) {
      const int e = e0 + 64 * r + lane;
      const uint32_t msk = s_um[e];
      const uint64_t bal = __ballot(msk != 0u);
      if (msk) {
        const uint32_t at = pos + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
        onodes[at] = (uint32_t)(c0 + e);
        omasks[at] = msk;
      }
      pos += (uint32_t)__popcll(bal);
    }
    if (chunk == nchunks - 1 && tid == kUnionThreads - 1) {
      uint32_t tot = before;
      for (int v = 0; v < NW; ++v) tot += wtot[v];
      cur.count[u] = tot;
    }
  }
  if (!sel_idx) return;
  for (int mm = wave + NW * zg; mm < Mu; mm += NW * ng) {
    const int qh = qh_of(geo, u, mm);
    const int anc = min(anchor, head_vis(geo, qh));  // the member's anchor tokens
    const int tok_base = (int)w.cut[4 * (int64_t)qh + 2];
    int32_t* sel = sel_idx + (int64_t)qh * cap;
    uint32_t mpos = wave_prefix_total(w.mcnt + (int64_t)qh * w.nuc, chunk, lane);
    uint32_t* stage = s_stage[wave];
    // the member's kept nodes of 8 x 64 entries, in order (ballots), then their tokens as
    // one run of 16-byte aligned stores (4-byte stores at its ends): 4 to 32 times fewer
    // store instructions than one token per lane per 64 entries (union and write 34.9 ->
    // 31.6 us at 256K deep; runs of 4 x 64 and 32 x 64 entries measured slower)
    for (int r0 = 0; r0 < kUnionChunk / 64; r0 += 8) {
      uint32_t n = 0;
#pragma unroll
      for (int r = r0; r < r0 + 8; ++r) {
        const int e = 64 * r + lane;
        const bool kept = (s_um[e] >> mm) & 1u;
        const uint64_t bal = __ballot(kept);
        if (kept) stage[n + __popcll(bal & ((1ull << lane) - 1ull))] = (uint32_t)(c0 + e);
        n += (uint32_t)__popcll(bal);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      write_token_run(sel + tok_base + (int64_t)mpos * b, (int)n * b, stage, geo.bdiv, anc, lane,
                      64);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      mpos += n;
    }
  }
}

// ---------------------------------------------------------------------------------- tail
// The tokens a head sees after its last complete top node (and after its anchor tokens)
// are attended like the anchor: appended to its ascending token list (after the level-1
// selection, which wrote tokens below them only) and to its count. Without a search the
// list is every token the head sees, and every level's union count is zeroed so that the
// per-level lists read as empty.
__global__ __launch_bounds__(256) void tail_kernel(Geom geo, int searched, int anchor,
                                                   int32_t* __restrict__ sel_idx,
                                                   int64_t cap, int32_t* __restrict__ sel_count,
                                                   uint32_t* __restrict__ counts,
                                                   int count_words) {
  const int qh = blockIdx.x;
  // the head's tail: after its last complete top node and its anchor tokens
  const int vis = head_vis(geo, qh);
  const int tail_lo =
      searched ? max((vis / geo.top_span) * geo.top_span, min(anchor, vis)) : 0;
  const int n_tail = vis - tail_lo;
  const int base = searched ? sel_count[qh] : 0;
  if (!searched && qh == 0)
    for (int i = threadIdx.x; i < count_words; i += 256) counts[i] = 0u;
  if (sel_idx) {
    int32_t* sel = sel_idx + (int64_t)qh * cap + base;
    for (int i = threadIdx.x; i < n_tail; i += 256) sel[i] = tail_lo + i;
  }
  __syncthreads();  // every thread has read the count
  if (threadIdx.x == 0) sel_count[qh] = base + n_tail;
}

// --------------------------------------------------------------------------- compaction
// The members' kept-flag rows are ORed into a member mask per frontier entry; entries with
// a non-empty mask, in ascending order, form the level's union list. The frontier is cut
// into chunks of kCompactChunk entries: a frontier of one chunk is compacted by one
// workgroup per unit; larger ones by a count launch (entries kept per chunk) and a write
// launch (each chunk adds the counts of the chunks before it), one workgroup per
// (unit, chunk) in both.

// Member masks of this thread's EPT entries c0 + EPT t .. (zero past F); returns count.
template <int EPT>
__device__ __forceinline__ uint32_t chunk_masks(const Geom& geo, int u, int Mu, int F, int c0,
                                                const KeepBits& kb, uint32_t (*sbits)[kCompactChunk / 32],
                                                uint32_t (&msk)[EPT]) {
  // stage the members' bit words of this chunk; every thread issues its loads together
  constexpr int kPer = kMaxMembers * (kCompactChunk / 32) / kCompactThreads;
  const int words = (min(kCompactChunk, F - c0) + 31) / 32;
  uint32_t v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = threadIdx.x + j * kCompactThreads;
    const int mm = i / (kCompactChunk / 32), wd = i % (kCompactChunk / 32);
    v[j] = (mm < Mu && wd < words)
               ? kb.bits[(int64_t)qh_of(geo, u, mm) * kb.words + c0 / 32 + wd] : 0u;
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = threadIdx.x + j * kCompactThreads;
    sbits[i / (kCompactChunk / 32)][i % (kCompactChunk / 32)] = v[j];
  }
  __syncthreads();
  const int e0 = EPT * threadIdx.x;
  uint32_t cnt = 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) msk[i] = 0u;
  if (c0 + e0 < F) {
    for (int mm = 0; mm < Mu; ++mm) {
      const uint32_t w = sbits[mm][e0 / 32] >> (e0 % 32);
#pragma unroll
      for (int i = 0; i < EPT; ++i) msk[i] |= ((w >> i) & 1u) << mm;
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      if (c0 + e0 + i >= F) msk[i] = 0u;
      cnt += msk[i] != 0u;
    }
  }
  return cnt;
}

// Writes this thread's kept entries from position r on. Node ids come from parent loads
// at indices clamped below F, issued together before any store.
template <int EPT>
__device__ __forceinline__ void chunk_write(int c0, uint32_t r, const uint32_t (&msk)[EPT],
                                            const LevelBufs& cur, int u) {
  const int e0 = EPT * threadIdx.x;  // entry c0 + e0 + i is node c0 + e0 + i
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    if (msk[i]) {
      cur.nodes[u * cur.stride + r] = (uint32_t)(c0 + e0 + i);
      cur.masks[u * cur.stride + r] = msk[i];
      ++r;
    }
  }
}

constexpr int kEPT = kCompactChunk / kCompactThreads;  // entries per thread (16)

// mode 0: one workgroup walks every chunk of the unit. mode 1: count chunk blockIdx.x into
// chunk_cnt. mode 2: write chunk blockIdx.x after the counts of the chunks before it.
__global__ __launch_bounds__(kCompactThreads) void compact_kernel(
    Geom geo, Frontier fr, KeepBits kb, LevelBufs cur, int mode, uint32_t* __restrict__ chunk_cnt,
    int max_chunks) {
  __shared__ uint32_t sbits[kMaxMembers][kCompactChunk / 32];
  __shared__ uint32_t wave_sum[kCompactThreads / 64];
  const int u = blockIdx.y;
  const int F = unit_entries(geo, fr, u);
  const int Mu = members_of(geo, u);
  uint32_t msk[kEPT];
  if (mode == 0) {
    uint32_t out = 0;
    for (int c0 = 0; c0 < F; c0 += kCompactChunk) {
      __syncthreads();
      const uint32_t cnt = chunk_masks<kEPT>(geo, u, Mu, F, c0, kb, sbits, msk);
      uint32_t total;
      const uint32_t r = out + block_excl_scan<kCompactThreads>(cnt, wave_sum, &total);
      chunk_write<kEPT>(c0, r, msk, cur, u);
      out += total;
    }
    if (threadIdx.x == 0) cur.count[u] = out;
    return;
  }
  const int chunk = blockIdx.x;
  const int c0 = chunk * kCompactChunk;
  const int nchunks = (F + kCompactChunk - 1) / kCompactChunk;
  if (c0 >= F) {
    if (mode == 1 && threadIdx.x == 0) chunk_cnt[u * max_chunks + chunk] = 0u;
    return;
  }
  const uint32_t cnt = chunk_masks<kEPT>(geo, u, Mu, F, c0, kb, sbits, msk);
  uint32_t total;
  const uint32_t r = block_excl_scan<kCompactThreads>(cnt, wave_sum, &total);
  if (mode == 1) {
    if (threadIdx.x == 0) chunk_cnt[u * max_chunks + chunk] = total;
    return;
  }
  uint32_t before = 0;
  for (int c = 0; c < chunk; ++c) before += chunk_cnt[u * max_chunks + c];
  chunk_write<kEPT>(c0, before + r, msk, cur, u);
  if (chunk == nchunks - 1 && threadIdx.x == 0) cur.count[u] = before + total;
}

}  // namespace

// Frontier entries per score workgroup (a multiple of 64: whole row groups for four waves).
// Measured at 256K deep: 1024 for the level-1 frontiers (64K entries per unit; 512 and
// 2048 were slower), 256 below (the 16K-entry level: 30 us against 35 us with 512).
int score_entries(int64_t cap_entries, int units) {
  (void)units;
  return cap_entries >= 65536 ? 1024 : 256;
}

hipError_t launch_score(const Geom& geo, const float* X, int64_t X_unit_stride, const void* Q,
                        int dtype, const Frontier& fr, float* S, int64_t S_stride,
                        const WideSel* wide, const uint8_t* rcodes, const uint8_t* rscales,
                        int64_t rows_cap, hipStream_t s) {
  if (fr.F < 1) return hipErrorInvalidValue;
  const int ent = score_entries(fr.F, geo.U);
  if (!rcodes && ent > kRowEntries) return hipErrorInvalidValue;
  dim3 grid((fr.F + ent - 1) / ent, geo.U);
  const float sigma = 1.0f / sqrtf((float)geo.D);
  float* pmax = wide ? wide->pmax : nullptr;
  float* pmin = wide ? wide->pmin : nullptr;
  const int64_t pstride = wide ? wide->pstride : 0;
#define ZHA_SCORE_FP4(DD, TQ)                                                           \
  hipLaunchKernelGGL((score_fp4_kernel<DD, TQ>), grid, dim3(kScoreThreads), 0, s, geo,       \
                     (const TQ*)Q, fr, S, S_stride, sigma, ent, pmax, pmin, pstride, rcodes,   \
                     rscales, rows_cap)
#define ZHA_ROWS(DD, TQ, MM, LL)                                                        \
  hipLaunchKernelGGL((score_rows_kernel<DD, TQ, MM, LL>), grid, dim3(kScoreThreads), 0, s, geo, \
                     X, X_unit_stride, (const TQ*)Q, fr, S, S_stride, sigma, ent, pmax, pmin,  \
                     pstride)
  // the float32 router scores with coalesced whole-row loads; the member count rounds up
  // to 8 or 16. Rows are split over 16 lanes (8 at d = 64 with 8 members), so every
  // exchange of the member butterfly is a DPP move within 16 lanes (with 32 lanes per row
  // the first exchange crosses rows through LDS: 0.84 against 0.59 ms for 16 members at
  // 256K)
  const bool m16 = geo.Tb * geo.G > 8;
#define ZHA_SCORE_D(DD, TQ)                                       \
  if (rcodes) ZHA_SCORE_FP4(DD, TQ);                              \
  else if (m16) ZHA_ROWS(DD, TQ, 16, 16);                         \
  else ZHA_ROWS(DD, TQ, 8, (DD) / 8)
  if (geo.D == 64) {
    if (dtype == ZHA_BF16) { ZHA_SCORE_D(64, bf16_t); }
    else { ZHA_SCORE_D(64, float); }
  } else {
    if (dtype == ZHA_BF16) { ZHA_SCORE_D(128, bf16_t); }
    else { ZHA_SCORE_D(128, float); }
  }
#undef ZHA_SCORE_D
#undef ZHA_ROWS
#undef ZHA_SCORE_FP4
  return hipGetLastError();
}

bool select_is_wide(int64_t cap_entries) { return cap_entries >= kWideMin; }
int64_t wide_partial_stride(int64_t cap_entries) {
  return (cap_entries + 255) / 256;  // the smallest score workgroup takes 256 entries
}
int64_t wide_chunks(int64_t cap_entries) { return (cap_entries + kWideChunk - 1) / kWideChunk; }
int64_t wide_union_chunks(int64_t cap_entries) {
  return (cap_entries + kUnionChunk - 1) / kUnionChunk;
}
int64_t wide_union_stride(int64_t cap_entries) {
  return wide_union_chunks(cap_entries) * kUnionChunk;
}
int wide_buckets() { return kWB; }

hipError_t launch_select(const Geom& geo, int level, const float* S, int64_t S_stride,
                         const Frontier& fr, KeepBits kb, float p, int anchor,
                         int32_t* sel_idx, int64_t cap, int32_t* sel_count, int32_t* lvl_kept,
                         const WideSel* wide, hipStream_t s) {
  const int QH = geo.B * geo.T * geo.Hq;
  if (fr.F < 1) return hipErrorInvalidValue;
  if (wide) {
    const dim3 grid((unsigned)((fr.F + kWideChunk - 1) / kWideChunk), QH);
    hipLaunchKernelGGL(wide_hist_kernel, grid, dim3(kWideThreads), 0, s, geo, S, S_stride, fr,
                       *wide);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (QH > kComputeUnits)
      hipLaunchKernelGGL(wide_cut_kernel<kCutThreads / 2>, dim3(QH), dim3(kCutThreads / 2), 0, s,
                         geo, level, S, S_stride, fr, kb, p, anchor, sel_idx, cap, sel_count,
                         lvl_kept, *wide);
    else
      hipLaunchKernelGGL(wide_cut_kernel<kCutThreads>, dim3(QH), dim3(kCutThreads), 0, s, geo,
                         level, S, S_stride, fr, kb, p, anchor, sel_idx, cap, sel_count,
                         lvl_kept, *wide);
    return hipGetLastError();
  }
  if (!kb.bits) return hipErrorInvalidValue;
  hipLaunchKernelGGL(select_kernel, dim3(QH), dim3(kSelThreads), 0, s, geo, level, S, S_stride,
                     fr, kb, p, anchor, sel_idx, cap, sel_count, lvl_kept);
  return hipGetLastError();
}

hipError_t launch_compact(const Geom& geo, const Frontier& fr, KeepBits kb, const LevelBufs& cur,
                          uint32_t* chunk_cnt, hipStream_t s) {
  const int F = fr.F;
  const int max_chunks = (F + kCompactChunk - 1) / kCompactChunk;
  if (max_chunks <= 1) {
    hipLaunchKernelGGL(compact_kernel, dim3(1, geo.U), dim3(kCompactThreads), 0, s, geo, fr, kb,
                       cur, 0, chunk_cnt, 1);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(compact_kernel, dim3(max_chunks, geo.U), dim3(kCompactThreads), 0, s, geo,
                     fr, kb, cur, 1, chunk_cnt, max_chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compact_kernel, dim3(max_chunks, geo.U), dim3(kCompactThreads), 0, s, geo,
                     fr, kb, cur, 2, chunk_cnt, max_chunks);
  return hipGetLastError();
}

int top_levels_lowest(const Geom& geo, const int64_t* nodes_per_level) {
  int lo = 0;
  for (int l = geo.L; l >= 2 && nodes_per_level[l] <= kTopFuse; --l) lo = l;
  return lo;  // 0: no level qualifies
}

hipError_t launch_top_levels(const Geom& geo, const float* pyramid, const int64_t* level_off,
                             const int64_t* unit_stride, int l_lo, const void* Q, int dtype,
                             float p, int32_t* lvl_kept, uint32_t* bitmaps,
                             const RouterView* router, hipStream_t s) {
  TopLevels tl{};
  for (int l = l_lo; l <= geo.L; ++l) {
    tl.xoff[l] = level_off[l];
    tl.xstride[l] = unit_stride[l];
  }
  const float sigma = 1.0f / sqrtf((float)geo.D);
  const int QH = geo.B * geo.T * geo.Hq;
  const RouterView rv = router ? *router : RouterView{};
  const int n_wg = geo.U * geo.Tb * geo.G;
  const bool half = n_wg > kComputeUnits;
#define ZHA_TOP_NT(DD, TQ, F4, NT)                                                            \
  hipLaunchKernelGGL((head_top_kernel<DD, TQ, F4, NT>), dim3(n_wg), dim3(NT), 0, s, geo,     \
                     pyramid, tl, geo.L, l_lo, (const TQ*)Q, p, sigma, lvl_kept, bitmaps, rv)
#define ZHA_TOP(DD, TQ, F4)                          \
  if (half) ZHA_TOP_NT(DD, TQ, F4, kTopThreads / 2); \
  else ZHA_TOP_NT(DD, TQ, F4, kTopThreads)
#define ZHA_TOP_D(DD, TQ)          \
  if (router) ZHA_TOP(DD, TQ, true); \
  else ZHA_TOP(DD, TQ, false)
  if (geo.D == 64) {
    if (dtype == ZHA_BF16) { ZHA_TOP_D(64, bf16_t); }
    else { ZHA_TOP_D(64, float); }
  } else {
    if (dtype == ZHA_BF16) { ZHA_TOP_D(128, bf16_t); }
    else { ZHA_TOP_D(128, float); }
  }
#undef ZHA_TOP_D
#undef ZHA_TOP
#undef ZHA_TOP_NT
  return hipGetLastError();
}

int64_t top_bitmap_words(int QH, int L) { return (int64_t)QH * (L + 1) * kTopWords; }
void top_level_layout(int L, int level, int64_t* word_off, int64_t* row_words) {
  *word_off = (int64_t)level * kTopWords;
  *row_words = (int64_t)(L + 1) * kTopWords;
}

hipError_t launch_tail(const Geom& geo, int searched, int anchor, int32_t* sel_idx,
                       int64_t cap, int32_t* sel_count, uint32_t* counts, int count_words,
                       hipStream_t s) {
  const int QH = geo.B * geo.T * geo.Hq;
  hipLaunchKernelGGL(tail_kernel, dim3(QH), dim3(256), 0, s, geo, searched, anchor, sel_idx,
                     cap, sel_count, counts, count_words);
  return hipGetLastError();
}

hipError_t launch_union(const Geom& geo, const float* S, int64_t S_stride, const Frontier& fr,
                        const LevelBufs& cur, int anchor, int32_t* sel_idx, int64_t cap,
                        const WideSel& wide, hipStream_t s) {
  if (fr.F < 1) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wide_union_chunks(fr.F), geo.U);
  hipLaunchKernelGGL(wide_union_kernel, grid, dim3(kUnionThreads), 0, s, geo, S, S_stride, fr,
                     wide);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the members' token lists are shared out over two workgroups per chunk
  const dim3 wgrid(grid.x, grid.y, sel_idx ? 2 : 1);
  hipLaunchKernelGGL(wide_write_kernel, wgrid, dim3(kUnionThreads), 0, s, geo, fr, cur, anchor,
                     sel_idx, cap, wide);
  return hipGetLastError();
}

// Chunk counters the compaction needs (uint32 entries) for a frontier of up to n entries.
int64_t compact_counter_words(int U, int64_t n) {
  return (int64_t)U * ((n + kCompactChunk - 1) / kCompactChunk);
}

}  // namespace zha
