/*
 * zha.h -- C ABI of the MI355X (gfx950) tree-indexed sparse decode attention library.
 *
 * Method: Zyphra Hierarchical Attention's tree-indexed sparse attention, as stated in
 * "Zyphra présente Zyphra Hierarchical Attention (ZHA), une voie vers une attention
 * vraiment sous-quadratique" (Le Fil IA, from MarkTechPost), paragraph 1: the full KV
 * cache is kept; keys are cut into contiguous blocks of b, each summarised by one
 * summary key obtained from 16 reference queries; summaries are grouped level by level
 * (b = 4 with 6 levels gives top nodes of 4,096 tokens); a decoding query scores the top
 * nodes, keeps the smallest set covering a fraction p of the estimated attention mass,
 * expands only those branches down to raw keys, always keeps the first token, and
 * attention runs over the gathered keys. Paragraph 2 of the same page fixes p = 0.95 and
 * the deep (b = 4, L = 6) and wide (b = 256, L = 1) geometries.
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument named as "device" is HIP device memory owned by the caller.
 *     The library allocates no device memory; its only state is a thread-local error
 *     string and, while launch timing is enabled, the recorded HIP events.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Entry points
 *     only enqueue work on it and never synchronise; device faults surface at the
 *     caller's next synchronisation.
 *   - Every argument check happens on the host before anything is enqueued; a negative
 *     zha_status is returned and zha_last_error() describes the problem.
 *   - Shapes are row-major. A KV cache is [B][Hkv][N_cap][d]: N_cap is its allocated
 *     length, and tokens [0, N) are in use.
 *   - K, V, Q, the reference queries, O and the pyramid must be 16-byte aligned and a
 *     workspace 256-byte aligned (hipMalloc returns 256-byte aligned memory); other
 *     pointers are rejected with ZHA_ERR_INVALID_ARG.
 *   - Supported: d in {64, 128}; dtype ZHA_F32 or ZHA_BF16 (K, V, Q and the reference
 *     queries share one dtype); b >= 2; 1 <= L <= ZHA_MAX_LEVELS; b^L <= 2^31;
 *     N_cap % b^L == 0 (any N <= N_cap); Hq % Hkv == 0 and Hq / Hkv <= 16;
 *     N_cap / b <= 2^21.
 */
#ifndef ZHA_H_
#define ZHA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ZHA_OK = 0,
  ZHA_ERR_INVALID_ARG = -1, /* null or misaligned pointer, p not in (0, 1], anchor out of
                               range, b < 2, L < 1, unknown router or no router copy */
  ZHA_ERR_SHAPE = -2,       /* b^L > 2^31, N_cap % b^L != 0, Hq % Hkv != 0, N > N_cap,
                               buffer too small */
  ZHA_ERR_DTYPE = -3,       /* unknown dtype */
  ZHA_ERR_CAPACITY = -4,    /* selected-list capacity smaller than N */
  ZHA_ERR_UNSUPPORTED = -5, /* d not in {64, 128}, Hq / Hkv > 16, L > ZHA_MAX_LEVELS, N / b > 2^21 */
  ZHA_ERR_HIP = -6          /* a HIP call or kernel launch failed */
} zha_status;

typedef enum { ZHA_F32 = 0, ZHA_BF16 = 1 } zha_dtype;

/*
 * Which copy of the summary keys the search scores (page 3, paragraph 4: a variant of the
 * router in FP4 was also tested). ZHA_ROUTER_F32: the float32 pyramid. ZHA_ROUTER_MXFP4:
 * an MXFP4 copy written by zha_router_quantize; the query is quantised the same way and
 * every node score is sigma times the float32-accumulated dot product of the two.
 */
typedef enum { ZHA_ROUTER_F32 = 0, ZHA_ROUTER_MXFP4 = 1 } zha_router;

#define ZHA_MAX_LEVELS 12
#define ZHA_N_REF 16 /* reference queries per KV head (page 3, paragraph 1) */

/*
 * Summary-key pyramid: a plain view of caller-owned device memory; nothing to free.
 * Level l (1..L) holds float32 summary keys [B][Hkv][N_cap / b^l][d] starting at
 * pyramid + level_off[l] (float elements). Node j of level l covers tokens
 * [j * b^l, (j + 1) * b^l) and exists once all of them are cached: with N cached tokens,
 * nodes 0 .. N / b^l - 1 (integer division) are valid. Levels are written by
 * zha_build_tree / zha_tree_append.
 *
 * MXFP4 router copy (zha_router_quantize): level l's node j, in unit u = b * Hkv + g, has
 * d / 2 code bytes at router_data + router_code_off[l] + (u * (N_cap / b^l) + j) * d / 2
 * (element 2i in the low nibble of byte i, element 2i + 1 in the high nibble; E2M1 codes:
 * sign bit 3, exponent bits 2..1 with bias 1, mantissa bit 0) and d / 32 scale bytes at
 * router_data + router_scale_off[l] + (u * (N_cap / b^l) + j) * d / 32 (E8M0: the block of
 * elements 32k .. 32k + 31 is scaled by 2^(byte - 127)). zha_build_tree sets router to
 * ZHA_ROUTER_F32 and router_data to NULL.
 *
 * The view is the library's: zha_build_tree writes the level offsets and
 * zha_router_quantize the router copy's. A caller may lower N to append tokens again (each
 * append re-pools the nodes it completes) and may switch router between the two copies;
 * N grows only through zha_tree_append. Every entry point that takes a tree checks its
 * fields, its geometry and that every offset is where the library puts it, and returns
 * ZHA_ERR_INVALID_ARG otherwise (a view filled by hand can be laid out by zha_build_tree
 * over zero tokens, which enqueues nothing).
 */
typedef struct {
  int32_t B, Hkv, N, N_cap, d, b, L;
  int32_t dtype;                              /* zha_dtype of the keys it was built from */
  int64_t level_off[ZHA_MAX_LEVELS + 1];      /* float offset of level l; [0] unused (= 0) */
  float* pyramid;                             /* device */
  int32_t router;                             /* zha_router: the copy zha_attend scores */
  int64_t router_code_off[ZHA_MAX_LEVELS + 1];  /* byte offsets into router_data */
  int64_t router_scale_off[ZHA_MAX_LEVELS + 1];
  uint8_t* router_data;                       /* device, or NULL: no MXFP4 copy */
} zha_tree;

/* Bytes of pyramid storage for a cache of capacity N_cap (0 if the geometry is invalid). */
size_t zha_tree_bytes(int B, int Hkv, int N_cap, int d, int b, int L);

/*
 * Build the pyramid over tokens [0, N) (page 3, paragraph 1: contiguous blocks of b, one
 * summary key per block from 16 reference queries, grouped level by level).
 *   K            device, dtype, [B][Hkv][N_cap][d]
 *   ref_queries  device, dtype, [Hkv][16][d]: one set per KV head, shared by all levels
 *   pyramid      device, at least zha_tree_bytes(B, Hkv, N_cap, d, b, L) bytes
 *   out          host; receives the view (N set to N)
 * Pooling: for each node, reference query r attends over the node's b children at scale
 * 1/sqrt(d); the 16 attention outputs are averaged into the node's summary key (a convex
 * combination of the children). Upper levels pool the stored level below the same way.
 * Summaries are float32 at every level.
 */
int zha_build_tree(const void* K, const void* ref_queries, int dtype, int B, int Hkv, int N,
                   int N_cap, int d, int b, int L, void* pyramid, size_t pyramid_bytes,
                   zha_tree* out, void* stream);

/* Bytes of MXFP4 router storage for a tree of this geometry (0 if the geometry is invalid). */
size_t zha_router_bytes(int B, int Hkv, int N_cap, int d, int b, int L);

/*
 * Write the MXFP4 copy of the pyramid the FP4 router scores (page 3, paragraph 4), and
 * select it: t->router = ZHA_ROUTER_MXFP4, t->router_data = router_data, offsets set.
 * Encodes, at every level l, the nodes complete at t->N tokens that were not complete at
 * n_from tokens (nodes [n_from / b^l, N / b^l); n_from = 0 encodes every node), from the
 * float32 pyramid, following OCP Microscaling Formats v1.0: per block of 32 elements,
 * X = floor(log2(max |x|)) - 2 (clamped to >= -127; -127 for an all-zero block), and each
 * element is x / 2^X rounded to the nearest E2M1 value (ties to the even mantissa) after
 * clamping to +-6, with the sign of x.
 *   router_data  device, 16-byte aligned, at least zha_router_bytes(...) bytes
 *   0 <= n_from <= t->N
 * Once a tree has a router copy, zha_tree_append encodes the nodes it completes. Setting
 * t->router back to ZHA_ROUTER_F32 makes zha_attend score the float32 pyramid again.
 */
int zha_router_quantize(zha_tree* t, int n_from, void* router_data, size_t router_bytes,
                        void* stream);

/*
 * Extend a tree by n_new >= 0 tokens (one at a time during generation, or in chunks):
 * pools, at every level, exactly the nodes the new tokens complete, then sets
 * t->N += n_new; t->N + n_new <= t->N_cap. A node's summary depends only on the tokens
 * under it, so any sequence of appends gives the pyramid one zha_build_tree over the same
 * tokens gives. K and ref_queries as for zha_build_tree (same cache, same reference
 * queries). With an MXFP4 router copy (t->router_data set), the new nodes are encoded too.
 */
int zha_tree_append(zha_tree* t, const void* K, const void* ref_queries, int n_new, void* stream);

/* Workspace bytes zha_attend needs for this tree and query shape (0 if invalid). */
size_t zha_attend_workspace_bytes(const zha_tree* t, int T, int Hq);

/*
 * Tree-indexed sparse decode attention (page 3, paragraph 1).
 *   t          tree built over the same K (its dtype, B, Hkv, N, N_cap, d)
 *   Q          device, dtype, [B][T][Hq][d]: T decode queries per sequence; query head h
 *              reads KV head h / (Hq / Hkv)
 *   K, V       device, dtype, [B][Hkv][N_cap][d]
 *   p          fraction of estimated attention mass to cover, in (0, 1]; p = 1 keeps all
 *   anchor     number of leading tokens always kept (the page's rule is 1; 0 disables),
 *              0 <= anchor <= N; added after the selection, outside the mass
 *   O          device, float32, [B][T][Hq][d]
 *   sel_idx    device, int32, [B][T][Hq][cap] or NULL: ascending selected token ids;
 *              entries past sel_count are left untouched
 *   cap        row length of sel_idx; must be >= N when sel_idx is not NULL
 *   sel_count  device, int32, [B][T][Hq]: number of selected tokens per query head
 *   workspace  device, at least zha_attend_workspace_bytes(t, T, Hq) bytes; its contents
 *              need no initialisation and are overwritten
 * Per query head: the top level's nodes form the first frontier; at each level the node
 * scores are sigma * q . X (sigma = 1/sqrt(d)), the estimated mass is their softmax over
 * the frontier, and the kept set is the shortest prefix of the frontier in order of
 * descending score (ties: lower node id first) whose mass reaches p; the next frontier
 * is the children of the kept nodes. The selected tokens are the b tokens of every kept
 * level-1 node plus tokens [0, anchor). The search runs over the complete top nodes
 * (N / b^L of them); the tail, tokens [(N / b^L) * b^L, N), is selected for every head
 * (with no complete top node, every token is). O is exact softmax attention at scale
 * sigma over the selected tokens, accumulated in float32. Calls that share a workspace
 * must not overlap. With t->router == ZHA_ROUTER_MXFP4 the node scores are computed from
 * the MXFP4 copy and the query quantised the same way (t->router_data must be set); the
 * final attention is unchanged.
 */
int zha_attend(const zha_tree* t, const void* Q, int T, int Hq, const void* K, const void* V,
               float p, int anchor, float* O, int32_t* sel_idx, int64_t cap,
               int32_t* sel_count, void* workspace, size_t ws_bytes, void* stream);

/*
 * zha_attend for T queries of each sequence that sit at their own positions, causally
 * masked (page 3, paragraph 3: a search that is itself sparse is what makes attention over
 * a whole sequence sub-quadratic).
 *   positions  device, int32, [B][T], 4-byte aligned: the 0-based position of query t of
 *              sequence b; values outside [0, N - 1] are clamped into it
 * The query at position t sees exactly the first t + 1 cached tokens, as if the cache
 * held only those: its search runs over the top nodes complete within them
 * ((t + 1) / b^L of them), its anchor is tokens [0, min(anchor, t + 1)), and the tokens it
 * sees after its last complete top node are selected; it never reads a later token. The
 * queries of one unit share one union list per level (each keeps its own set). Every
 * other argument, output and rule is that of zha_attend; with every position at N - 1 the
 * result is zha_attend's.
 */
int zha_attend_causal(const zha_tree* t, const void* Q, int T, int Hq, const int32_t* positions,
                      const void* K, const void* V, float p, int anchor, float* O,
                      int32_t* sel_idx, int64_t cap, int32_t* sel_count, void* workspace,
                      size_t ws_bytes, void* stream);

/*
 * zha_attend without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The workspace is a fixed device array of ZHA_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends; the current device's copy
 * (hipGetDevice; `stream` must belong to that device) is used. The call allocates nothing.
 * Every argument, output and rule is that of zha_attend. Errors: ZHA_ERR_CAPACITY when
 * zha_attend_workspace_bytes(t, T, Hq) exceeds ZHA_NOALLOC_SCRATCH_BYTES (checked on the
 * host before anything is enqueued; e.g. 256K tokens, 4 sequences, 32/4 heads, d = 128,
 * b = 4, L = 6 need about 77 MiB and fit, a 1M-token batch of 8 does not). All calls on
 * one GPU share its scratch: calls that overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller. The scratch needs no clearing; each
 * call overwrites what it reads.
 */
#define ZHA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int zha_attend_noalloc(const zha_tree* t, const void* Q, int T, int Hq, const void* K,
                       const void* V, float p, int anchor, float* O, int32_t* sel_idx,
                       int64_t cap, int32_t* sel_count, void* stream);

/*
 * Dense comparator: exact softmax attention of every query head over all N cached keys of
 * its KV head, with the same decode and combine kernels zha_attend uses (every member
 * reads every token; there is no tree and no search). It is what the tree-indexed path is
 * measured against (page 3, paragraph 4: the pages' speedups are relative to dense
 * attention). Q, K, V, O and the workspace as for zha_attend; the shapes are given
 * directly. 1 <= N <= N_cap, N <= 2^21, d in {64, 128}, Hq % Hkv == 0, Hq / Hkv <= 16.
 * zha_dense_workspace_bytes returns 0 for an invalid shape.
 */
size_t zha_dense_workspace_bytes(int B, int Hkv, int N, int N_cap, int d, int T, int Hq);
int zha_dense_attend(const void* Q, int T, int Hq, const void* K, const void* V, int dtype,
                     int B, int Hkv, int N, int N_cap, int d, float* O, void* workspace,
                     size_t ws_bytes, void* stream);

/* The dense comparator with query positions (as for zha_attend_causal): each query
 * attends exactly to tokens [0, position]. positions: device, int32, [B][T], non-NULL. */
int zha_dense_attend_causal(const void* Q, int T, int Hq, const int32_t* positions,
                            const void* K, const void* V, int dtype, int B, int Hkv, int N,
                            int N_cap, int d, float* O, void* workspace, size_t ws_bytes,
                            void* stream);

/*
 * Diagnostics of the last zha_attend that used `workspace` (valid once it completed).
 * The G = Hq / Hkv heads of one KV head (and up to 16 / G queries of one sequence) form a
 * "unit" that shares one union frontier per level: unit u = ((b * Hkv + g) * nTB + tb),
 * with Tb = min(T, 16 / G) queries per unit, nTB = ceil(T / Tb); member
 * m = (t % Tb) * G + h % G. Level 1 (the list the decode reads) is kept as a union list;
 * this reports byte offsets into the workspace of:
 *   nodes  uint32 [U][stride]: ascending ids of the level-1 nodes kept by any member
 *   masks  uint32 [U][stride]: bit m set when member m kept that node
 *   count  uint32 [U]:         number of valid entries per unit
 * and the number of units U through *units. level must be 1 (ZHA_ERR_INVALID_ARG
 * otherwise).
 */
int zha_attend_level_view(const zha_tree* t, int T, int Hq, int level, int64_t* off_nodes,
                          int64_t* off_masks, int64_t* off_count, int64_t* stride,
                          int64_t* units);

/*
 * The nodes each query head kept at level `level` in 2..L, as bits by node id: row qh
 * (qh = (b * T + t) * Hq + h) is *words uint32 words starting at byte offset
 * *off_bits + 4 * qh * *words of the workspace; bit j of the row (word j / 32, bit j % 32)
 * is set when head qh kept node j. Nodes 0 .. *nodes - 1 (those under the complete top
 * nodes; none when the cache holds no complete top node) are valid. Same validity as
 * zha_attend_level_view.
 */
int zha_attend_level_bits(const zha_tree* t, int T, int Hq, int level, int64_t* off_bits,
                          int64_t* words, int64_t* nodes);

/*
 * Per-launch timing (for benchmarks and profiling). While enabled, every kernel this
 * library launches is bracketed by two HIP events recorded on the launch's stream;
 * zha_timing_enable(1) starts a fresh record and zha_timing_enable(0) stops recording.
 * zha_timing_read waits for the recorded events and returns, for one kernel kind and
 * pyramid level (level = -1: every level), the summed duration in milliseconds and the
 * number of launches. Kinds: ZHA_K_POOL (pooling; the level is the first level a launch
 * writes, level 1 reads the keys), ZHA_K_SCORE, ZHA_K_SELECT, ZHA_K_COMPACT (per level),
 * ZHA_K_DECODE and ZHA_K_COMBINE (level 0), ZHA_K_DESCENT (the one launch that runs the
 * top levels whose frontiers hold at most 1024 entries; its level is the lowest of them).
 * Recording creates HIP events (host-side objects), so it is off by default.
 */
enum {
  ZHA_K_POOL = 0,
  ZHA_K_SCORE = 2,
  ZHA_K_SELECT = 3,
  ZHA_K_DECODE = 4,
  ZHA_K_COMPACT = 5,
  ZHA_K_COMBINE = 6,
  ZHA_K_DESCENT = 7,
  ZHA_K_ROUTER = 8 /* MXFP4 encoding of pyramid rows (level 0: every level of one call) */
};
int zha_timing_enable(int on);
int zha_timing_read(int kind, int level, double* total_ms, int64_t* launches);

/* Thread-local description of the last failing call on this thread ("" if none). */
const char* zha_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZHA_H_ */
