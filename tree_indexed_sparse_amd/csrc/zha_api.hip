// Host entry points of the C ABI declared in include/zha.h: argument checks, workspace
// layout and the launch sequence. Nothing here allocates device memory or synchronises.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "zha_internal.h"

using namespace zha;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(ZHA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ------------------------------------------------------------------ launch timing
struct TimedLaunch {
  int kind, level;
  hipEvent_t start, stop;
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<TimedLaunch> g_launches;
std::vector<hipEvent_t> g_free_events;

hipEvent_t take_event() {
  if (!g_free_events.empty()) {
    hipEvent_t e = g_free_events.back();
    g_free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Run `launch` (which enqueues one kernel on s); bracket it with events when timing is on.
template <class F>
hipError_t timed(int kind, int level, hipStream_t s, F&& launch) {
  std::unique_lock<std::mutex> lk(g_tmu);
  if (!g_timing) {
    lk.unlock();
    return launch();
  }
  TimedLaunch t{kind, level, take_event(), take_event()};
  if (t.start) hipEventRecord(t.start, s);
  const hipError_t e = launch();
  if (t.stop) hipEventRecord(t.stop, s);
  if (t.start && t.stop) g_launches.push_back(t);
  return e;
}

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int64_t ipow(int64_t b, int e) {
  int64_t r = 1;
  for (int i = 0; i < e; ++i) r *= b;
  return r;
}

// Checks shared by the tree entry points. Returns ZHA_OK or an error code (message set).
int check_geometry(int B, int Hkv, int N, int N_cap, int d, int b, int L) {
  if (B < 1 || Hkv < 1) return fail(ZHA_ERR_SHAPE, "B and Hkv must be >= 1 (got %d, %d)", B, Hkv);
  if (b < 2) return fail(ZHA_ERR_INVALID_ARG, "branching factor b must be >= 2 (got %d)", b);
  if (L < 1) return fail(ZHA_ERR_INVALID_ARG, "levels L must be >= 1 (got %d)", L);
  if (L > ZHA_MAX_LEVELS)
    return fail(ZHA_ERR_UNSUPPORTED, "levels L must be <= %d (got %d)", ZHA_MAX_LEVELS, L);
  if (d != 64 && d != 128) return fail(ZHA_ERR_UNSUPPORTED, "head dim must be 64 or 128 (got %d)", d);
  // b^L, stopping as soon as it passes 2^31 (each factor is below 2^31, so no product
  // overflows 64 bits)
  int64_t top = 1;
  for (int i = 0; i < L; ++i) {
    top *= b;
    if (top > (int64_t)1 << 31)
      return fail(ZHA_ERR_SHAPE, "b^L = %d^%d exceeds 2^31 tokens per top node", b, L);
  }
  if (N_cap < 1 || N_cap % top != 0)
    return fail(ZHA_ERR_SHAPE, "cache capacity N_cap=%d must be a positive multiple of b^L=%lld",
                N_cap, (long long)top);
  if (N < 0 || N > N_cap) return fail(ZHA_ERR_SHAPE, "N=%d must lie in [0, N_cap=%d]", N, N_cap);
  if (N_cap / b > (1 << kMaxLog2Nodes))
    return fail(ZHA_ERR_UNSUPPORTED, "N_cap / b must be <= 2^%d", kMaxLog2Nodes);
  return ZHA_OK;
}

// Workspace of zha_attend: every offset is in bytes and 256-byte aligned.
// Workspace of one attend call. Level 1 keeps a compacted union list (nodes, masks,
// count); every level l >= 2 keeps its member masks uncompacted, by node id (masks[l],
// written by the score launch one level down), and the members' kept bits (bits[l], or the
// fused descent's bitmaps for the levels it walks).
struct WsLayout {
  int U, QH, splits;
  int64_t n[ZHA_MAX_LEVELS + 1];  // nodes per unit at each level (current N)
  int64_t off_count, off_lvl, off_S, off_part, off_chunks;
  int64_t off_pmax, off_pmin, off_hm, off_hc, off_cut, off_umask, off_ucnt, off_mcnt, off_tbits;
  int64_t pstride, nch, ustride, nuc;
  int64_t off_nodes1, off_masks[ZHA_MAX_LEVELS + 1];
  int64_t off_bits[ZHA_MAX_LEVELS + 1], bit_words[ZHA_MAX_LEVELS + 1];
  int64_t S_stride;
  int64_t total;
};

int make_geom(const zha_tree* t, int T, int Hq, Geom* g) {
  if (T < 1 || Hq < 1) return fail(ZHA_ERR_SHAPE, "T and Hq must be >= 1 (got %d, %d)", T, Hq);
  if (Hq % t->Hkv != 0)
    return fail(ZHA_ERR_SHAPE, "Hq=%d must be a multiple of Hkv=%d", Hq, t->Hkv);
  const int G = Hq / t->Hkv;
  if (G > kMaxMembers)
    return fail(ZHA_ERR_UNSUPPORTED, "Hq / Hkv = %d exceeds %d", G, kMaxMembers);
  // query heads are numbered in int32 (kernel indices, workspace rows)
  if ((int64_t)t->B * T * Hq > INT32_MAX)
    return fail(ZHA_ERR_UNSUPPORTED, "B * T * Hq = %lld query heads exceeds 2^31 - 1",
                (long long)t->B * T * Hq);
  g->B = t->B;
  g->T = T;
  g->Hq = Hq;
  g->Hkv = t->Hkv;
  g->G = G;
  g->Tb = T < kMaxMembers / G ? T : kMaxMembers / G;
  g->nTB = (T + g->Tb - 1) / g->Tb;
  g->U = t->B * t->Hkv * g->nTB;
  g->D = t->d;
  g->b = t->b;
  g->L = t->L;
  g->N = t->N;
  g->Ncap = t->N_cap;
  g->bdiv = make_fastdiv((uint32_t)t->b);
  g->top_span = (int)ipow(t->b, t->L);
  g->pos = nullptr;
  return ZHA_OK;
}

WsLayout layout_of(const Geom& g) {
  WsLayout w{};
  w.U = g.U;
  w.QH = g.B * g.T * g.Hq;
  w.splits = decode_splits(g.U, g.pos != nullptr);
  int64_t nl = g.N;
  for (int l = 1; l <= g.L; ++l) {
    nl /= g.b;
    w.n[l] = nl;
  }
  int64_t off = 0;
  w.off_count = off;
  off = align256(off + 4 * (int64_t)(g.L + 1) * g.U);
  w.off_lvl = off;
  off = align256(off + 4 * (int64_t)w.QH * (g.L + 1));
  for (int l = 1; l <= g.L; ++l) {
    const int64_t bytes = 4 * (int64_t)g.U * w.n[l];
    if (l == 1) {
      w.off_nodes1 = off;
      off = align256(off + bytes);
    }
    w.off_masks[l] = off;
    off = align256(off + bytes);
    w.bit_words[l] = (w.n[l] + 31) / 32;
    w.off_bits[l] = off;
    off = align256(off + 4 * (int64_t)w.QH * w.bit_words[l]);
  }
  w.S_stride = (w.n[1] + 3) / 4 * 4;  // score rows start 16-byte aligned
  w.off_S = off;
  off = align256(off + 4 * (int64_t)w.QH * w.S_stride);
  w.off_part = off;
  off = align256(off + 4 * (int64_t)g.U * decode_splits(g.U, true) * kMaxMembers * (g.D + 2));
  w.off_chunks = off;
  off = align256(off + 4 * compact_counter_words(g.U, w.n[1]));
  // chunked-selection scratch, sized for the largest frontier (level 1)
  w.pstride = wide_partial_stride(w.n[1]);
  w.nch = wide_chunks(w.n[1]);
  w.off_pmax = off;
  off = align256(off + 4 * (int64_t)w.QH * w.pstride);
  w.off_pmin = off;
  off = align256(off + 4 * (int64_t)w.QH * w.pstride);
  w.off_hm = off;
  off = align256(off + 8 * (int64_t)w.QH * w.nch * wide_buckets());
  w.off_hc = off;
  off = align256(off + 4 * (int64_t)w.QH * w.nch * wide_buckets());
  w.off_cut = off;
  off = align256(off + 16 * (int64_t)w.QH);
  w.ustride = wide_union_stride(w.n[1]);
  w.nuc = wide_union_chunks(w.n[1]);
  w.off_umask = off;
  off = align256(off + 4 * (int64_t)g.U * w.ustride);
  w.off_ucnt = off;
  off = align256(off + 4 * (int64_t)g.U * w.nuc);
  w.off_mcnt = off;
  off = align256(off + 4 * (int64_t)w.QH * w.nuc);
  w.off_tbits = off;
  off = align256(off + 4 * top_bitmap_words(w.QH, g.L));
  w.total = off;
  return w;
}

// level 1's union list
LevelBufs level1_bufs(char* ws, const WsLayout& w) {
  LevelBufs lb;
  lb.nodes = (uint32_t*)(ws + w.off_nodes1);
  lb.masks = (uint32_t*)(ws + w.off_masks[1]);
  lb.count = (uint32_t*)(ws + w.off_count) + w.U;
  lb.stride = w.n[1];
  return lb;
}

// The kept bits of level l: the fused descent's bitmaps for l >= l_top > 0. Byte offset
// into the workspace and words per query head.
void level_bits_at(const WsLayout& w, int L, int l_top, int l, int64_t* off, int64_t* words) {
  if (l_top && l >= l_top) {
    int64_t word_off;
    top_level_layout(L, l, &word_off, words);
    *off = w.off_tbits + 4 * word_off;
    return;
  }
  *off = w.off_bits[l];
  *words = w.bit_words[l];
}
KeepBits level_bits(char* ws, const WsLayout& w, int L, int l_top, int l) {
  int64_t off, words;
  level_bits_at(w, L, l_top, l, &off, &words);
  return KeepBits{(uint32_t*)(ws + off), words};
}

// Float offsets of the pyramid levels (level l at level_off[l], each level 256-byte
// aligned) for a valid geometry. Returns the total bytes.
int64_t pyramid_layout(int B, int Hkv, int N_cap, int d, int b, int L, int64_t* level_off) {
  int64_t off = 0, nl = N_cap;
  for (int l = 1; l <= L; ++l) {
    nl /= b;
    if (level_off) level_off[l] = off / 4;
    off = align256(off + 4 * (int64_t)B * Hkv * nl * d);
  }
  return off;
}

// Byte offsets of the MXFP4 router copy: per level the codes, then the scales, each
// 256-byte aligned. Returns the total size.
int64_t router_layout(int B, int Hkv, int N_cap, int d, int b, int L, int64_t* code_off,
                      int64_t* scale_off) {
  int64_t off = 0, nl = N_cap;
  for (int l = 1; l <= L; ++l) {
    nl /= b;
    const int64_t rows = (int64_t)B * Hkv * nl;
    if (code_off) code_off[l] = off;
    off = align256(off + rows * (d / 2));
    if (scale_off) scale_off[l] = off;
    off = align256(off + rows * (d / 32));
  }
  return off;
}

// A tree view as zha_build_tree (and zha_router_quantize) lay it out: valid fields and
// geometry, and every level's offset (and the router copy's, if attached) where the
// library puts it, so that no kernel is handed a pointer outside the caller's buffers.
int check_tree(const zha_tree* t) {
  if (!t) return fail(ZHA_ERR_INVALID_ARG, "tree is NULL");
  if (!t->pyramid) return fail(ZHA_ERR_INVALID_ARG, "tree has no pyramid");
  if (t->dtype != ZHA_F32 && t->dtype != ZHA_BF16)
    return fail(ZHA_ERR_DTYPE, "unknown dtype %d", t->dtype);
  if (t->router != ZHA_ROUTER_F32 && t->router != ZHA_ROUTER_MXFP4)
    return fail(ZHA_ERR_INVALID_ARG, "unknown router %d", t->router);
  if (t->router == ZHA_ROUTER_MXFP4 && !t->router_data)
    return fail(ZHA_ERR_INVALID_ARG, "router is MXFP4 but the tree has no router copy");
  const int st = check_geometry(t->B, t->Hkv, t->N, t->N_cap, t->d, t->b, t->L);
  if (st != ZHA_OK) return st;
  int64_t lo[ZHA_MAX_LEVELS + 1] = {0};
  pyramid_layout(t->B, t->Hkv, t->N_cap, t->d, t->b, t->L, lo);
  for (int l = 1; l <= t->L; ++l)
    if (t->level_off[l] != lo[l])
      return fail(ZHA_ERR_INVALID_ARG,
                  "tree level_off[%d] = %lld where zha_build_tree puts the level at %lld: "
                  "the view was not made (or was changed) outside the library",
                  l, (long long)t->level_off[l], (long long)lo[l]);
  if (t->router_data) {
    int64_t co[ZHA_MAX_LEVELS + 1] = {0}, so[ZHA_MAX_LEVELS + 1] = {0};
    router_layout(t->B, t->Hkv, t->N_cap, t->d, t->b, t->L, co, so);
    for (int l = 1; l <= t->L; ++l)
      if (t->router_code_off[l] != co[l] || t->router_scale_off[l] != so[l])
        return fail(ZHA_ERR_INVALID_ARG,
                    "tree router offsets of level %d (%lld, %lld) are not where "
                    "zha_router_quantize puts them (%lld, %lld)",
                    l, (long long)t->router_code_off[l], (long long)t->router_scale_off[l],
                    (long long)co[l], (long long)so[l]);
  }
  return ZHA_OK;
}

// Encode, at every level not marked in `skip`, rows [n_lo / b^l, n_hi / b^l) of each unit
// into the router copy.
hipError_t encode_router(const zha_tree* t, int64_t n_lo, int64_t n_hi, hipStream_t s,
                         const bool* skip = nullptr) {
  RouterJob job{};
  const int rpw = router_rows_per_workgroup(t->d);
  int wgs = 0;
  int64_t cap = t->N_cap, div = 1;
  for (int l = 1; l <= t->L; ++l) {
    cap /= t->b;
    div *= t->b;
    const int r0 = (int)(n_lo / div), r1 = (int)(n_hi / div);
    if (r1 <= r0 || (skip && skip[l])) continue;
    const int i = job.n++;
    job.src[i] = t->pyramid + t->level_off[l];
    job.codes[i] = t->router_data + t->router_code_off[l];
    job.scales[i] = t->router_data + t->router_scale_off[l];
    job.rows_cap[i] = cap;
    job.row0[i] = r0;
    job.row1[i] = r1;
    job.wg0[i] = wgs;
    wgs += (r1 - r0 + rpw - 1) / rpw;
  }
  if (job.n == 0) return hipSuccess;
  return timed(ZHA_K_ROUTER, 0, s, [&] {
    return launch_router_encode(job, t->B * t->Hkv, t->d, wgs, s);
  });
}

}  // namespace

extern "C" {

const char* zha_last_error(void) { return g_err.c_str(); }

size_t zha_tree_bytes(int B, int Hkv, int N_cap, int d, int b, int L) {
  const std::string saved = g_err;
  const int st = check_geometry(B, Hkv, 0, N_cap, d, b, L);
  g_err = saved;
  if (st != ZHA_OK) return 0;
  return (size_t)pyramid_layout(B, Hkv, N_cap, d, b, L, nullptr);
}

size_t zha_router_bytes(int B, int Hkv, int N_cap, int d, int b, int L) {
  const std::string saved = g_err;
  const int st = check_geometry(B, Hkv, 0, N_cap, d, b, L);
  g_err = saved;
  if (st != ZHA_OK) return 0;
  return (size_t)router_layout(B, Hkv, N_cap, d, b, L, nullptr, nullptr);
}

int zha_router_quantize(zha_tree* t, int n_from, void* router_data, size_t router_bytes,
                        void* stream) {
  if (!t) return fail(ZHA_ERR_INVALID_ARG, "tree is NULL");
  if (!router_data) return fail(ZHA_ERR_INVALID_ARG, "router_data must not be NULL");
  if (!aligned16(router_data))
    return fail(ZHA_ERR_INVALID_ARG, "router_data must be 16-byte aligned");
  zha_tree v = *t;  // checked as it will be once the copy is attached
  v.router = ZHA_ROUTER_MXFP4;
  v.router_data = (uint8_t*)router_data;
  // the geometry first (the router layout divides by b), then the copy's offsets as the
  // library lays them, then the whole view
  int st = check_geometry(v.B, v.Hkv, v.N, v.N_cap, v.d, v.b, v.L);
  if (st != ZHA_OK) return st;
  const int64_t need = router_layout(v.B, v.Hkv, v.N_cap, v.d, v.b, v.L, v.router_code_off,
                                     v.router_scale_off);
  st = check_tree(&v);
  if (st != ZHA_OK) return st;
  if (n_from < 0 || n_from > t->N)
    return fail(ZHA_ERR_SHAPE, "n_from=%d must lie in [0, N=%d]", n_from, t->N);
  if ((int64_t)router_bytes < need)
    return fail(ZHA_ERR_SHAPE, "router buffer has %zu bytes, needs %lld", router_bytes,
                (long long)need);
  const hipError_t e = encode_router(&v, n_from, v.N, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "router encode launch");
  *t = v;
  return ZHA_OK;
}

int zha_tree_append(zha_tree* t, const void* K, const void* R, int n_new, void* stream) {
  int st = check_tree(t);
  if (st != ZHA_OK) return st;
  if (!K || !R) return fail(ZHA_ERR_INVALID_ARG, "K and ref_queries must not be NULL");
  if (!aligned16(K) || !aligned16(R))
    return fail(ZHA_ERR_INVALID_ARG, "K and ref_queries must be 16-byte aligned");
  if (n_new < 0) return fail(ZHA_ERR_SHAPE, "n_new=%d must be >= 0", n_new);
  if ((int64_t)t->N + n_new > t->N_cap)
    return fail(ZHA_ERR_SHAPE, "N + n_new = %lld exceeds N_cap=%d", (long long)t->N + n_new,
                t->N_cap);
  hipStream_t s = (hipStream_t)stream;
  const int units = t->B * t->Hkv;
  // level l has N_cap / b^l nodes of capacity per (sequence, KV head)
  auto cap_nodes = [&](int l) { return (int64_t)t->N_cap / ipow(t->b, l); };
  // Nodes of level j that the append completes: [N_old / b^j, N_new / b^j). A fused launch
  // pools whole tiles of b^k child rows (k levels) that contain such nodes, with the
  // child rows cached so far as its limit: it stores every complete node of those tiles
  // (re-pooling a node that was already complete rewrites the same value, with the same
  // arithmetic) and none that is incomplete. Any sequence of appends therefore writes the
  // pyramid a one-shot build writes.
  const int64_t n_old = t->N, n_end = (int64_t)t->N + n_new;
  auto lo = [&](int j) { return n_old / ipow(t->b, j); };
  auto hi = [&](int j) { return n_end / ipow(t->b, j); };
  // levels whose router rows the pooling launches encode themselves
  bool encoded[ZHA_MAX_LEVELS + 1] = {false};
  for (int l = 1; l <= t->L;) {
    const void* child = (l == 1) ? K : (const void*)(t->pyramid + t->level_off[l - 1]);
    const int dt_in = (l == 1) ? t->dtype : ZHA_F32;
    const int k = fused_levels(t->b, t->L - l + 1);
    hipError_t e = hipSuccess;
    if (hi(l) > lo(l)) {
      if (k >= 1) {
        const int64_t tr = ipow(t->b, k);  // child rows (level l - 1) per tile
        const int64_t rows = hi(l - 1);    // child rows cached after the append
        const int64_t r0 = (lo(l - 1) / tr) * tr, r1 = (rows + tr - 1) / tr * tr;
        float* outs[ZHA_MAX_LEVELS];
        int64_t strides[ZHA_MAX_LEVELS];
        uint8_t* rc[ZHA_MAX_LEVELS];
        uint8_t* rs[ZHA_MAX_LEVELS];
        for (int j = 0; j < k; ++j) {
          outs[j] = t->pyramid + t->level_off[l + j];
          strides[j] = cap_nodes(l + j) * t->d;
          if (t->router_data) {
            rc[j] = t->router_data + t->router_code_off[l + j];
            rs[j] = t->router_data + t->router_scale_off[l + j];
          }
        }
        const bool enc = t->router_data &&
                         pool_fused_encodes(dt_in, t->dtype, t->b, k, (int)r0, (int)r1);
        for (int j = 0; j < k && enc; ++j) encoded[l + j] = true;
        e = timed(ZHA_K_POOL, l, s, [&] {
          return launch_pool_fused(dt_in, child, cap_nodes(l - 1) * t->d, R, t->dtype, outs,
                                   strides, k, units, t->Hkv, (int)r0, (int)r1, (int)rows, t->b,
                                   t->d, enc ? rc : nullptr, enc ? rs : nullptr, s);
        });
      } else {
        e = timed(ZHA_K_POOL, l, s, [&] {
          return launch_pool_level(dt_in, child, cap_nodes(l - 1) * t->d, R, t->dtype,
                                   t->pyramid + t->level_off[l], cap_nodes(l) * t->d, units,
                                   t->Hkv, (int)lo(l), (int)hi(l), t->b, t->d, s);
        });
      }
    }
    if (e != hipSuccess) return hip_fail(e, "pooling launch");
    l += k >= 1 ? k : 1;
  }
  if (t->router_data) {
    const hipError_t e = encode_router(t, n_old, n_end, s, encoded);
    if (e != hipSuccess) return hip_fail(e, "router encode launch");
  }
  t->N += n_new;
  return ZHA_OK;
}

int zha_build_tree(const void* K, const void* R, int dtype, int B, int Hkv, int N, int N_cap,
                   int d, int b, int L, void* pyramid, size_t pyramid_bytes, zha_tree* out,
                   void* stream) {
  if (!K || !R || !pyramid || !out)
    return fail(ZHA_ERR_INVALID_ARG, "K, ref_queries, pyramid and out must not be NULL");
  if (!aligned16(K) || !aligned16(R) || !aligned16(pyramid))
    return fail(ZHA_ERR_INVALID_ARG, "K, ref_queries and pyramid must be 16-byte aligned");
  if (dtype != ZHA_F32 && dtype != ZHA_BF16) return fail(ZHA_ERR_DTYPE, "unknown dtype %d", dtype);
  int st = check_geometry(B, Hkv, N, N_cap, d, b, L);
  if (st != ZHA_OK) return st;
  const size_t need = zha_tree_bytes(B, Hkv, N_cap, d, b, L);
  if (pyramid_bytes < need)
    return fail(ZHA_ERR_SHAPE, "pyramid buffer has %zu bytes, needs %zu", pyramid_bytes, need);
  zha_tree t;
  memset(&t, 0, sizeof(t));
  t.B = B;
  t.Hkv = Hkv;
  t.N = 0;
  t.N_cap = N_cap;
  t.d = d;
  t.b = b;
  t.L = L;
  t.dtype = dtype;
  t.pyramid = (float*)pyramid;
  pyramid_layout(B, Hkv, N_cap, d, b, L, t.level_off);
  st = zha_tree_append(&t, K, R, N, stream);
  if (st != ZHA_OK) return st;
  *out = t;
  return ZHA_OK;
}

size_t zha_attend_workspace_bytes(const zha_tree* t, int T, int Hq) {
  const std::string saved = g_err;
  Geom g;
  int st = check_tree(t);
  if (st == ZHA_OK) st = make_geom(t, T, Hq, &g);
  g_err = saved;
  if (st != ZHA_OK || t->N == 0) return 0;
  return (size_t)layout_of(g).total;
}

// ---- dense comparator: the decode kernels over every cached key, no search
namespace {
struct DenseLayout {
  int64_t off_part, total;
  int splits;
};
int dense_geom(int B, int Hkv, int N, int N_cap, int d, int T, int Hq, Geom* g) {
  if (B < 1 || Hkv < 1) return fail(ZHA_ERR_SHAPE, "B and Hkv must be >= 1 (got %d, %d)", B, Hkv);
  if (d != 64 && d != 128) return fail(ZHA_ERR_UNSUPPORTED, "head dim must be 64 or 128 (got %d)", d);
  if (N < 1 || N > N_cap) return fail(ZHA_ERR_SHAPE, "N=%d must lie in [1, N_cap=%d]", N, N_cap);
  if (N > (1 << kMaxLog2Nodes))
    return fail(ZHA_ERR_UNSUPPORTED, "N=%d must be <= 2^%d", N, kMaxLog2Nodes);
  zha_tree t{};
  t.B = B;
  t.Hkv = Hkv;
  t.N = N;
  t.N_cap = N_cap;
  t.d = d;
  t.b = 2;
  t.L = 1;
  return make_geom(&t, T, Hq, g);
}
DenseLayout dense_layout(const Geom& g) {
  DenseLayout w{};
  w.splits = decode_splits(g.U, g.pos != nullptr);
  w.off_part = 0;
  w.total = align256(4 * (int64_t)g.U * decode_splits(g.U, true) * kMaxMembers * (g.D + 2));
  return w;
}
}  // namespace

size_t zha_dense_workspace_bytes(int B, int Hkv, int N, int N_cap, int d, int T, int Hq) {
  const std::string saved = g_err;
  Geom g;
  const int st = dense_geom(B, Hkv, N, N_cap, d, T, Hq, &g);
  g_err = saved;
  if (st != ZHA_OK) return 0;
  return (size_t)dense_layout(g).total;
}

namespace {
int dense_impl(const void* Q, int T, int Hq, const int32_t* positions, const void* K,
               const void* V, int dtype, int B, int Hkv, int N, int N_cap, int d, float* O,
               void* workspace, size_t ws_bytes, void* stream) {
  if (!Q || !K || !V || !O || !workspace)
    return fail(ZHA_ERR_INVALID_ARG, "Q, K, V, O and workspace must not be NULL");
  if (dtype != ZHA_F32 && dtype != ZHA_BF16) return fail(ZHA_ERR_DTYPE, "unknown dtype %d", dtype);
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) ||
      ((uintptr_t)workspace & 255u) != 0)
    return fail(ZHA_ERR_INVALID_ARG,
                "Q, K, V and O must be 16-byte aligned and the workspace 256-byte aligned");
  if (positions && ((uintptr_t)positions & 3u) != 0)
    return fail(ZHA_ERR_INVALID_ARG, "positions must be 4-byte aligned");
  Geom g;
  int st = dense_geom(B, Hkv, N, N_cap, d, T, Hq, &g);
  if (st != ZHA_OK) return st;
  g.pos = positions;
  const DenseLayout w = dense_layout(g);
  if ((int64_t)ws_bytes < w.total)
    return fail(ZHA_ERR_SHAPE, "workspace has %zu bytes, needs %lld", ws_bytes,
                (long long)w.total);
  hipStream_t s = (hipStream_t)stream;
  float* part = (float*)((char*)workspace + w.off_part);
  // no list: every token a member sees is its tail
  hipError_t e = timed(ZHA_K_DECODE, 0, s, [&] {
    return launch_decode(g, dtype, K, V, Q, LevelBufs{}, 0, 0, w.splits, part, s);
  });
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  e = timed(ZHA_K_COMBINE, 0, s, [&] { return launch_combine(g, w.splits, part, O, s); });
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return ZHA_OK;
}
}  // namespace

int zha_dense_attend(const void* Q, int T, int Hq, const void* K, const void* V, int dtype,
                     int B, int Hkv, int N, int N_cap, int d, float* O, void* workspace,
                     size_t ws_bytes, void* stream) {
  return dense_impl(Q, T, Hq, nullptr, K, V, dtype, B, Hkv, N, N_cap, d, O, workspace, ws_bytes,
                    stream);
}

int zha_dense_attend_causal(const void* Q, int T, int Hq, const int32_t* positions,
                            const void* K, const void* V, int dtype, int B, int Hkv, int N,
                            int N_cap, int d, float* O, void* workspace, size_t ws_bytes,
                            void* stream) {
  if (!positions) return fail(ZHA_ERR_INVALID_ARG, "positions must not be NULL");
  return dense_impl(Q, T, Hq, positions, K, V, dtype, B, Hkv, N, N_cap, d, O, workspace,
                    ws_bytes, stream);
}

int zha_attend_level_view(const zha_tree* t, int T, int Hq, int level, int64_t* off_nodes,
                          int64_t* off_masks, int64_t* off_count, int64_t* stride,
                          int64_t* units) {
  int st = check_tree(t);
  if (st != ZHA_OK) return st;
  Geom g;
  st = make_geom(t, T, Hq, &g);
  if (st != ZHA_OK) return st;
  if (level != 1)
    return fail(ZHA_ERR_INVALID_ARG,
                "level %d: only level 1 keeps a union list (zha_attend_level_bits has the "
                "levels above)", level);
  if (!off_nodes || !off_masks || !off_count || !stride || !units)
    return fail(ZHA_ERR_INVALID_ARG, "output pointers must not be NULL");
  const WsLayout w = layout_of(g);
  *off_nodes = w.off_nodes1;
  *off_masks = w.off_masks[1];
  *off_count = w.off_count + 4 * (int64_t)w.U;
  *stride = w.n[1];
  *units = w.U;
  return ZHA_OK;
}

int zha_attend_level_bits(const zha_tree* t, int T, int Hq, int level, int64_t* off_bits,
                          int64_t* words, int64_t* nodes) {
  int st = check_tree(t);
  if (st != ZHA_OK) return st;
  Geom g;
  st = make_geom(t, T, Hq, &g);
  if (st != ZHA_OK) return st;
  if (level < 2 || level > t->L)
    return fail(ZHA_ERR_INVALID_ARG, "level %d outside [2, %d]", level, t->L);
  if (!off_bits || !words || !nodes)
    return fail(ZHA_ERR_INVALID_ARG, "output pointers must not be NULL");
  const WsLayout w = layout_of(g);
  const int64_t n_top = w.n[t->L];
  const int l_top = n_top > 0 ? top_levels_lowest(g, w.n) : 0;
  level_bits_at(w, t->L, l_top, level, off_bits, words);
  *nodes = n_top * ipow(t->b, t->L - level);
  return ZHA_OK;
}

namespace {
int attend_impl(const zha_tree* t, const void* Q, int T, int Hq, const int32_t* positions,
                const void* K, const void* V, float p, int anchor, float* O, int32_t* sel_idx,
                int64_t cap, int32_t* sel_count, void* workspace, size_t ws_bytes,
                void* stream) {
  int st = check_tree(t);
  if (st != ZHA_OK) return st;
  if (!Q || !K || !V || !O || !sel_count || !workspace)
    return fail(ZHA_ERR_INVALID_ARG, "Q, K, V, O, sel_count and workspace must not be NULL");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) ||
      ((uintptr_t)workspace & 255u) != 0)
    return fail(ZHA_ERR_INVALID_ARG,
                "Q, K, V and O must be 16-byte aligned and the workspace 256-byte aligned");
  if (t->N < 1) return fail(ZHA_ERR_SHAPE, "the tree covers no tokens");
  if (!(p > 0.0f && p <= 1.0f)) return fail(ZHA_ERR_INVALID_ARG, "p=%g must lie in (0, 1]", (double)p);
  if (anchor < 0 || anchor > t->N)
    return fail(ZHA_ERR_INVALID_ARG, "anchor=%d must lie in [0, N=%d]", anchor, t->N);
  if (sel_idx && cap < t->N)
    return fail(ZHA_ERR_CAPACITY, "sel_idx row length cap=%lld is smaller than N=%d",
                (long long)cap, t->N);
  if (positions && ((uintptr_t)positions & 3u) != 0)
    return fail(ZHA_ERR_INVALID_ARG, "positions must be 4-byte aligned");
  Geom g;
  st = make_geom(t, T, Hq, &g);
  if (st != ZHA_OK) return st;
  g.pos = positions;
  const WsLayout w = layout_of(g);
  if ((int64_t)ws_bytes < w.total)
    return fail(ZHA_ERR_SHAPE, "workspace has %zu bytes, needs %lld", ws_bytes,
                (long long)w.total);

  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const LevelBufs lv1 = level1_bufs(ws, w);
  float* S = (float*)(ws + w.off_S);
  int32_t* lvl = (int32_t*)(ws + w.off_lvl);
  WideSel wsel;
  wsel.pmax = (float*)(ws + w.off_pmax);
  wsel.pmin = (float*)(ws + w.off_pmin);
  wsel.pstride = w.pstride;
  wsel.hm = (unsigned long long*)(ws + w.off_hm);
  wsel.hc = (uint32_t*)(ws + w.off_hc);
  wsel.nch = w.nch;
  wsel.cut = (uint32_t*)(ws + w.off_cut);
  wsel.umask = (uint32_t*)(ws + w.off_umask);
  wsel.ustride = w.ustride;
  wsel.ucnt = (uint32_t*)(ws + w.off_ucnt);
  wsel.mcnt = (uint32_t*)(ws + w.off_mcnt);
  wsel.nuc = w.nuc;

  hipError_t e = hipSuccess;
  int64_t unit_stride[ZHA_MAX_LEVELS + 1] = {0};  // pyramid floats per (sequence, KV head)
  {
    int64_t c = t->N_cap;
    for (int l = 1; l <= t->L; ++l) {
      c /= t->b;
      unit_stride[l] = c * t->d;
    }
  }
  // The search runs over the complete top nodes; the tail (tokens after the last of them)
  // is attended by every head. With no complete top node the whole cache is the tail.
  const int n_top_nodes = (int)w.n[t->L];
  const bool searched = n_top_nodes > 0;
  const int64_t n_full = (int64_t)n_top_nodes * ipow(t->b, t->L);
  const int tail_lo = searched ? (int)std::max<int64_t>(n_full, anchor) : 0;
  const int n_tail = t->N - tail_lo;
  // FP4 router: every level is scored from the MXFP4 copy
  const bool fp4 = t->router == ZHA_ROUTER_MXFP4;
  RouterView rv{};
  if (fp4) {
    for (int l = 1; l <= t->L; ++l) {
      rv.codes[l] = t->router_data + t->router_code_off[l];
      rv.scales[l] = t->router_data + t->router_scale_off[l];
    }
  }
  // the top levels with small frontiers run fused in one launch
  const int l_top = searched ? top_levels_lowest(g, w.n) : 0;
  if (l_top) {
    e = timed(ZHA_K_DESCENT, l_top, s, [&] {
      return launch_top_levels(g, t->pyramid, t->level_off, unit_stride, l_top, Q, t->dtype, p,
                               lvl, (uint32_t*)(ws + w.off_tbits), fp4 ? &rv : nullptr, s);
    });
    if (e != hipSuccess) return hip_fail(e, "top-level descent launch");
  }
  int64_t cap_l = t->N_cap;
  for (int l = 1; l <= t->L; ++l) cap_l /= t->b;  // capacity nodes at the top level
  for (int l = l_top ? l_top - 1 : t->L; l < t->L; ++l) cap_l *= t->b;
  int64_t F = n_top_nodes;  // frontier entries at level l: its nodes under the top nodes
  for (int l = l_top ? l_top - 1 : t->L; l < t->L; ++l) F *= t->b;
  for (int l = l_top ? l_top - 1 : t->L; searched && l >= 1; --l) {
    Frontier fr{};
    fr.F = (int)F;
    fr.span = (int)ipow(t->b, t->L - l);
    if (l < t->L) {
      const KeepBits pb = level_bits(ws, w, t->L, l_top, l + 1);
      fr.pbits = pb.bits;
      fr.pwords = pb.words;
      fr.pmask = (uint32_t*)(ws + w.off_masks[l + 1]);
      fr.pstride = w.n[l + 1];
    }
    const float* X = t->pyramid + t->level_off[l];
    wsel.pent = score_entries(F, g.U);
    const WideSel* wide = select_is_wide(F) ? &wsel : nullptr;
    // the kept bits the level below reads (level 1: the narrow selection's, for its
    // compaction; the chunked one compacts from the scores and cuts)
    const KeepBits kb = (l > 1 || !wide) ? level_bits(ws, w, t->L, l_top, l) : KeepBits{};
    e = timed(ZHA_K_SCORE, l, s, [&] {
      return launch_score(g, X, cap_l * t->d, Q, t->dtype, fr, S, w.S_stride, wide,
                          fp4 ? rv.codes[l] : nullptr, fp4 ? rv.scales[l] : nullptr, cap_l, s);
    });
    if (e != hipSuccess) return hip_fail(e, "score launch");
    e = timed(ZHA_K_SELECT, l, s, [&] {
      return launch_select(g, l, S, w.S_stride, fr, kb, p, anchor, l == 1 ? sel_idx : nullptr,
                           cap, sel_count, lvl, wide, s);
    });
    if (e != hipSuccess) return hip_fail(e, "select launch");
    if (l == 1) {
      e = timed(ZHA_K_COMPACT, l, s, [&] {
        if (wide)
          return launch_union(g, S, w.S_stride, fr, lv1, anchor, sel_idx, cap, *wide, s);
        return launch_compact(g, fr, kb, lv1, (uint32_t*)(ws + w.off_chunks), s);
      });
      if (e != hipSuccess) return hip_fail(e, "compact launch");
    }
    cap_l *= t->b;
    F *= t->b;
  }
  if (!searched || n_tail > 0 || positions) {
    e = timed(ZHA_K_SELECT, 0, s, [&] {
      return launch_tail(g, searched ? 1 : 0, anchor, sel_idx, cap, sel_count,
                         (uint32_t*)(ws + w.off_count), (t->L + 1) * g.U, s);
    });
    if (e != hipSuccess) return hip_fail(e, "tail launch");
  }
  float* part = (float*)(ws + w.off_part);
  e = timed(ZHA_K_DECODE, 0, s, [&] {
    return launch_decode(g, t->dtype, K, V, Q, lv1, searched ? 1 : 0, searched ? anchor : 0,
                         w.splits, part, s);
  });
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  e = timed(ZHA_K_COMBINE, 0, s, [&] { return launch_combine(g, w.splits, part, O, s); });
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return ZHA_OK;
}
}  // namespace

int zha_attend(const zha_tree* t, const void* Q, int T, int Hq, const void* K, const void* V,
               float p, int anchor, float* O, int32_t* sel_idx, int64_t cap, int32_t* sel_count,
               void* workspace, size_t ws_bytes, void* stream) {
  return attend_impl(t, Q, T, Hq, nullptr, K, V, p, anchor, O, sel_idx, cap, sel_count,
                     workspace, ws_bytes, stream);
}

int zha_attend_causal(const zha_tree* t, const void* Q, int T, int Hq, const int32_t* positions,
                      const void* K, const void* V, float p, int anchor, float* O,
                      int32_t* sel_idx, int64_t cap, int32_t* sel_count, void* workspace,
                      size_t ws_bytes, void* stream) {
  if (!positions) return fail(ZHA_ERR_INVALID_ARG, "positions must not be NULL");
  return attend_impl(t, Q, T, Hq, positions, K, V, p, anchor, O, sel_idx, cap, sel_count,
                     workspace, ws_bytes, stream);
}

}  // extern "C"

// ------------------------------------------------------------- allocation-free attend
// The workspace of zha_attend_noalloc: a file-scope device array that each GPU holds for
// the life of the process. Host code never uses the array's name as an address (on the
// host it is only a stand-in for the symbol); the per-device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
namespace {
static __device__ __align__(256) unsigned char scratch[ZHA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ZHA_ERR_UNSUPPORTED, "device %d outside the %d devices the scratch serves", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(ZHA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ZHA_OK;
}
}  // namespace

extern "C" {

int zha_attend_noalloc(const zha_tree* t, const void* Q, int T, int Hq, const void* K,
                       const void* V, float p, int anchor, float* O, int32_t* sel_idx,
                       int64_t cap, int32_t* sel_count, void* stream) {
  int st = check_tree(t);
  if (st != ZHA_OK) return st;
  Geom g;
  st = make_geom(t, T, Hq, &g);
  if (st != ZHA_OK) return st;
  if (t->N >= 1) {
    const int64_t need = layout_of(g).total;
    if (need > (int64_t)ZHA_NOALLOC_SCRATCH_BYTES)
      return fail(ZHA_ERR_CAPACITY,
                  "zha_attend_noalloc: this tree and query shape need %lld bytes of workspace, "
                  "more than the %lld-byte device scratch; use zha_attend with a workspace",
                  (long long)need, (long long)ZHA_NOALLOC_SCRATCH_BYTES);
  }
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != ZHA_OK) return st;
  return attend_impl(t, Q, T, Hq, nullptr, K, V, p, anchor, O, sel_idx, cap, sel_count, ws,
                     (size_t)ZHA_NOALLOC_SCRATCH_BYTES, stream);
}

int zha_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (on) {
    for (auto& t : g_launches) {
      g_free_events.push_back(t.start);
      g_free_events.push_back(t.stop);
    }
    g_launches.clear();
  }
  g_timing = on != 0;
  return ZHA_OK;
}

int zha_timing_read(int kind, int level, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return fail(ZHA_ERR_INVALID_ARG, "output pointers must not be NULL");
  std::lock_guard<std::mutex> lk(g_tmu);
  double tot = 0.0;
  int64_t n = 0;
  for (auto& t : g_launches) {
    if (t.kind != kind || (level >= 0 && t.level != level)) continue;
    hipError_t e = hipEventSynchronize(t.stop);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, t.start, t.stop);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return ZHA_OK;
}

}  // extern "C"
