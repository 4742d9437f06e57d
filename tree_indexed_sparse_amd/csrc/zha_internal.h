// Internal definitions shared by the gfx950 kernels and the host entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zha.h"

namespace zha {

constexpr int kNRef = ZHA_N_REF;   // reference queries per KV head
constexpr int kMaxMembers = 16;    // query heads (x queries) sharing one union list
constexpr int kMaxLog2Nodes = 21;  // frontier bound that keeps 2^42-scaled masses in u64
constexpr int kMaxSplits = 128;    // decode splits per unit (partials merged in one workgroup)

constexpr int kComputeUnits = 256;  // MI355X: 8 XCDs of 32 CUs

// Decode workgroups per launch: three per compute unit. Two are resident per CU at a
// time, and the launch takes as long as its busiest CU's share of the K/V bytes, so the
// count is a multiple of the CU count and the splits are equal.
constexpr int kDecodeWorkgroups = 3 * kComputeUnits;

// Decode splits per unit for U units: every unit gets the same number and the total stays
// at or below kDecodeWorkgroups (no CU takes a fourth workgroup). With query positions the
// units' work differs (each sees its own prefix of the cache): there the pieces are finer
// (about 4096 workgroups), so that the dispatch of workgroups to free CUs evens it out.
// The positioned count is never the smaller one; the workspace is sized for it.
inline int decode_splits(int U, bool positioned) {
  const int u = U > 0 ? U : 1;
  int s = kDecodeWorkgroups / u;
  if (positioned && 4096 / u > s) s = 4096 / u;
  return s < 1 ? 1 : (s > kMaxSplits ? kMaxSplits : s);
}

typedef uint16_t bf16_t;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// Division by a runtime constant d >= 1 for numerators below 2^31 (round-up magic
// number): q = (mulhi(n, m) + n) >> l with l = ceil(log2 d), m = 2^32 (2^l - d) / d + 1.
// The GPU has no integer divider; this replaces ~30 instructions by three.
struct FastDiv {
  uint32_t d, m, l;
  __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
    return (__umulhi(n, m) + n) >> l;
  }
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  FastDiv f;
  f.d = d;
  f.l = l;
  f.m = (uint32_t)((((1ull << 32) * ((1ull << l) - d)) / d) + 1);
  return f;
}

// Decode-call geometry. A unit is (sequence, KV head, block of Tb queries); its members
// are the Tb * G (query, head) pairs that read that KV head.
struct Geom {
  int B, T, Hq, Hkv, G, Tb, nTB, U;
  int D, b, L, N, Ncap;
  FastDiv bdiv;  // division by b
  int top_span;        // b^L: tokens under one top node
  const int32_t* pos;  // [B][T] query positions, or null: every query sees all N tokens
};

__host__ __device__ __forceinline__ int members_of(const Geom& g, int u) {
  const int tb = u % g.nTB;
  const int rem = g.T - tb * g.Tb;
  return (rem < g.Tb ? rem : g.Tb) * g.G;
}

// query head index qh = (bb * T + t) * Hq + h  <->  (unit, member)
__host__ __device__ __forceinline__ void unit_member_of(const Geom& g, int qh, int* u, int* m) {
  const int h = qh % g.Hq;
  const int t = (qh / g.Hq) % g.T;
  const int bb = qh / (g.Hq * g.T);
  const int kv = h / g.G, j = h % g.G;
  const int tb = t / g.Tb, tl = t % g.Tb;
  *u = (bb * g.Hkv + kv) * g.nTB + tb;
  *m = tl * g.G + j;
}

__host__ __device__ __forceinline__ int qh_of(const Geom& g, int u, int m) {
  const int tb = u % g.nTB;
  const int kv = (u / g.nTB) % g.Hkv;
  const int bb = u / (g.nTB * g.Hkv);
  const int t = tb * g.Tb + m / g.G;
  const int h = kv * g.G + m % g.G;
  return (bb * g.T + t) * g.Hq + h;
}

// Tokens query head qh sees: its position + 1 (positions clamped into [0, N - 1]), or N
// without positions. Its search runs over the top nodes complete within them.
__device__ __forceinline__ int head_vis(const Geom& g, int qh) {
  if (!g.pos) return g.N;
  const int t = (qh / g.Hq) % g.T, bb = qh / (g.Hq * g.T);
  const int p = g.pos[bb * g.T + t];
  return (p < 0 ? 0 : (p >= g.N ? g.N - 1 : p)) + 1;
}
__device__ __forceinline__ int head_ntop(const Geom& g, int qh) {
  return head_vis(g, qh) / g.top_span;
}

// (sequence, KV head) index of a unit: selects the K/V/pyramid slice.
__host__ __device__ __forceinline__ int bg_of(const Geom& g, int u) { return u / g.nTB; }

// Per-level union lists in the workspace.
struct LevelBufs {
  uint32_t* nodes;   // [U][stride] kept node ids (ascending)
  uint32_t* masks;   // [U][stride] member bitmask per kept node
  uint32_t* count;   // [U]
  int64_t stride;    // = nodes at this level
};

// Per-query-head kept flags of one level, by node id (bit j of row qh: head qh kept node j).
struct KeepBits {
  uint32_t* bits;    // [QH][words]
  int64_t words;
};

// The frontier a level is searched over, indexed by node id: entry k is node k of the
// level. Below the top it holds the children of every node of the level above; entry k
// belongs to member m's frontier when m kept its parent k / b (entries whose parent no
// member kept are skipped, not compacted away). At the top level (pbits null) it is the
// complete top nodes, each member's own the first head_ntop of them.
struct Frontier {
  const uint32_t* pbits;  // [QH][pwords]: the level above's kept bits; null at the top
  int64_t pwords;
  uint32_t* pmask;        // [U][pstride]: member mask per parent node (bit m: member m kept
  int64_t pstride;        //   it), written by the level's score launch, read after it
  int F;                  // entries: the level's nodes under the complete top nodes
  int span;               // nodes of this level under one top node (b^(L - l))
};

// unit u's member masks per parent node (null at the top)
__host__ __device__ __forceinline__ const uint32_t* parent_masks(const Frontier& fr, int u) {
  return fr.pbits ? fr.pmask + (int64_t)u * fr.pstride : nullptr;
}

// Entries of member qh's frontier lie below this: the nodes under the top nodes complete
// for it (with query positions a member sees a prefix of the cache).
__device__ __forceinline__ int member_entries(const Geom& g, const Frontier& fr, int qh) {
  return min(fr.F, head_ntop(g, qh) * fr.span);
}
// Entries of unit u's frontier lie below this: the largest of its members' bounds, which
// depend only on the positions of the unit's queries (tb Tb .. of sequence bb).
__device__ __forceinline__ int unit_entries(const Geom& g, const Frontier& fr, int u) {
  if (!g.pos) return fr.F;
  const int tb = u % g.nTB, bb = u / (g.nTB * g.Hkv);
  const int t0 = tb * g.Tb, t1 = min(g.T, t0 + g.Tb);
  int vis = 0;
  for (int t = t0; t < t1; ++t) {
    const int p = g.pos[bb * g.T + t];
    vis = max(vis, (p < 0 ? 0 : (p >= g.N ? g.N - 1 : p)) + 1);
  }
  return min(fr.F, (vis / g.top_span) * fr.span);
}

// Scratch of the chunked selection and compaction that large frontiers take (workgroups
// over frontier chunks instead of one per query head or unit).
struct WideSel {
  float* pmax;                // [QH][pstride] member max score per score workgroup
  float* pmin;                // [QH][pstride] member min score per score workgroup
  int64_t pstride;
  int pent;                   // frontier entries per score workgroup at this level
  unsigned long long* hm;     // [QH][nch][buckets] fixed-point mass per chunk and bucket
  uint32_t* hc;               // [QH][nch][buckets] entry count per chunk and bucket
  int64_t nch;
  uint32_t* cut;              // [QH][4] cut score bits, cut index, token base, kept total
  uint32_t* umask;            // [U][ustride] member mask per frontier entry (uncompacted)
  int64_t ustride;
  uint32_t* ucnt;             // [U][nuc] union entries per compaction chunk
  uint32_t* mcnt;             // [QH][nuc] member's kept entries per compaction chunk
  int64_t nuc;
};

// MXFP4 copy of the pyramid that the FP4 router scores (codes: d / 2 bytes per node, two
// elements per byte, low nibble first; scales: d / 32 E8M0 bytes per node).
struct RouterView {
  const uint8_t* codes[ZHA_MAX_LEVELS + 1];   // level l base, [B*Hkv][N_cap / b^l][d / 2]
  const uint8_t* scales[ZHA_MAX_LEVELS + 1];  // level l base, [B*Hkv][N_cap / b^l][d / 32]
};

// One router-encoding launch: rows [row0, row1) of every (sequence, KV head) at each of
// n levels; workgroups wg0[i] .. wg0[i + 1] - 1 take level i.
struct RouterJob {
  const float* src[ZHA_MAX_LEVELS];
  uint8_t* codes[ZHA_MAX_LEVELS];
  uint8_t* scales[ZHA_MAX_LEVELS];
  int64_t rows_cap[ZHA_MAX_LEVELS];  // rows per (sequence, KV head) of the level's storage
  int row0[ZHA_MAX_LEVELS], row1[ZHA_MAX_LEVELS], wg0[ZHA_MAX_LEVELS];
  int n;
};

// ---------------------------------------------------------------------------------------
// launchers (defined in the .hip files; all enqueue on `s`, return hipGetLastError())
// ---------------------------------------------------------------------------------------

// One pyramid level: children [B*Hkv][*][D] (in_unit_stride elements apart) -> out.
hipError_t launch_pool_level(int dtype_in, const void* child, int64_t in_unit_stride,
                             const void* R, int dtype_r, float* out, int64_t out_unit_stride,
                             int units, int Hkv, int node_begin, int node_end, int b, int D,
                             hipStream_t s);

// Levels that one fused tile launch pools for branching factor b (0 if b > 64).
int fused_levels(int b, int levels_left);

// `nlev` consecutive levels pooled from one child level in one launch (b^nlev <= 64):
// child rows [row_begin, row_end) -> outs[j] (level j + 1 above the child level).
// rcodes / rscales (per fused level, or null): the MXFP4 router copy of those levels,
// written by the launch only when pool_fused_encodes() says so for its arguments.
hipError_t launch_pool_fused(int dtype_in, const void* child, int64_t in_unit_stride,
                             const void* R, int dtype_r, float* const* outs,
                             const int64_t* out_unit_strides, int nlev, int units, int Hkv,
                             int row_begin, int row_end, int row_limit, int b, int D,
                             uint8_t* const* rcodes, uint8_t* const* rscales, hipStream_t s);
bool pool_fused_encodes(int dtype_in, int dtype_r, int b, int nlev, int row_begin,
                        int row_end);

// Scores of a level's union frontier for every member: S[qh][k].
// wide != nullptr: also write the per-workgroup member max/min the chunked selection reads.
// rcodes != nullptr: score the level's MXFP4 copy (rcodes / rscales, rows_cap rows per
// unit) with the query quantised to MXFP4, instead of the float32 rows X.
hipError_t launch_score(const Geom& geo, const float* X, int64_t X_unit_stride, const void* Q,
                        int dtype, const Frontier& fr, float* S, int64_t S_stride,
                        const WideSel* wide, const uint8_t* rcodes, const uint8_t* rscales,
                        int64_t rows_cap, hipStream_t s);

// Whether a frontier of up to `cap_entries` entries takes the chunked selection, and the
// sizes of its scratch for frontiers up to `cap_entries`.
bool select_is_wide(int64_t cap_entries);
int64_t wide_partial_stride(int64_t cap_entries);
int score_entries(int64_t cap_entries, int units);  // frontier entries per score workgroup
int64_t wide_chunks(int64_t cap_entries);      // histogram chunks
int64_t wide_union_chunks(int64_t cap_entries);  // compaction chunks
int64_t wide_union_stride(int64_t cap_entries);  // umask row length
int wide_buckets();

// Per-member top-p: the kept flags into `kb` (by node id; the chunked selection writes
// them only when kb.bits is set); at level 1 also the token lists and counts.
hipError_t launch_select(const Geom& geo, int level, const float* S, int64_t S_stride,
                         const Frontier& fr, KeepBits kb, float p, int anchor,
                         int32_t* sel_idx, int64_t cap, int32_t* sel_count, int32_t* lvl_kept,
                         const WideSel* wide, hipStream_t s);

// Union of the members' kept flags -> ascending kept-node list with member masks.
// chunk_cnt: scratch of compact_counter_words(U, frontier capacity) words.
hipError_t launch_compact(const Geom& geo, const Frontier& fr, KeepBits kb, const LevelBufs& cur,
                          uint32_t* chunk_cnt, hipStream_t s);

// Fused descent through the top levels (frontiers of at most 1024 entries): the lowest
// such level >= 2 (0 if none; the top level must qualify), and the launch that walks
// levels L .. l_lo per query head and writes each level's kept bits into `bitmaps`
// (top_bitmap_words(QH, L) words; top_level_bits gives a level's rows).
int top_levels_lowest(const Geom& geo, const int64_t* nodes_per_level);
// router != nullptr: the levels are scored from the MXFP4 copy.
hipError_t launch_top_levels(const Geom& geo, const float* pyramid, const int64_t* level_off,
                             const int64_t* unit_stride, int l_lo, const void* Q, int dtype,
                             float p, int32_t* lvl_kept, uint32_t* bitmaps,
                             const RouterView* router, hipStream_t s);
int64_t top_bitmap_words(int QH, int L);
// level `level`'s bitmaps: row qh starts at word word_off + qh * row_words
void top_level_layout(int L, int level, int64_t* word_off, int64_t* row_words);

// Compaction after the chunked selection at level 1: the members' keep flags straight
// from their scores and cuts, the union list and the token lists.
hipError_t launch_union(const Geom& geo, const float* S, int64_t S_stride, const Frontier& fr,
                        const LevelBufs& cur, int anchor, int32_t* sel_idx, int64_t cap,
                        const WideSel& wide, hipStream_t s);
int64_t compact_counter_words(int U, int64_t n);

// Sparse GQA decode: the tokens of the level-1 union list (has_list), the anchor tokens
// [0, min(anchor, seen)) and each member's tail: the tokens it sees after its last
// complete top node (has_list), or every token it sees (no list: dense attention).
hipError_t launch_decode(const Geom& geo, int dtype, const void* K, const void* V,
                         const void* Q, const LevelBufs& l1, int has_list, int anchor,
                         int splits, float* partials, hipStream_t s);

// Appends each head's tail (the tokens it sees after its last complete top node and the
// anchor) to its token list and count, after the level-1 selection wrote them; searched =
// 0: the list is every token the head sees, and every level's union count is zeroed.
hipError_t launch_tail(const Geom& geo, int searched, int anchor, int32_t* sel_idx,
                       int64_t cap, int32_t* sel_count, uint32_t* counts, int count_words,
                       hipStream_t s);

// MXFP4 encoding of pyramid rows (the FP4 router's copy), every level of `job` at once.
int router_rows_per_workgroup(int D);
hipError_t launch_router_encode(const RouterJob& job, int units, int D, int workgroups,
                                hipStream_t s);

// Merge the decode partials of every split, in split order, into O.
hipError_t launch_combine(const Geom& geo, int splits, const float* partials, float* O,
                          hipStream_t s);

}  // namespace zha
