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
#include "zha_mxfp4.h"

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

// ------------------------------------------------------------------------------------
// Fused tile pooling for b <= 64: a workgroup stages TR = b^k child rows in LDS and pools
// k consecutive levels from them (TR <= 64), so the child level is read once and every
// pooled level is written once. The 16 x d reference-query contraction runs on the matrix
// cores: v_mfma_f32_16x16x32_bf16 when the children are bf16 keys (products exact in
// fp32), v_mfma_f32_16x16x4_f32 for float32 summaries. One 16-row block per wave:
// A = 16 child rows (read from LDS), B = R^T (held in registers), C = z^T[row][ref].
// The softmax over each node's children, the mean over reference queries and the
// weighted sum of the children run on the vector units in fixed orders.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTileRows = 64;
constexpr int kMaxFuse = 6;  // 2^6 = 64 rows
constexpr int kTilesPerWG = 1;

struct PoolOut {
  float* ptr[kMaxFuse];
  int64_t unit_stride[kMaxFuse];
  // MXFP4 router copy of the same levels (null: none): codes [unit][rows][D/2] and scales
  // [unit][rows][D/32], rows = unit_stride / D
  uint8_t* codes[kMaxFuse];
  uint8_t* scales[kMaxFuse];
};

__device__ __forceinline__ uint4 lds16(const uint32_t* p) { return *reinterpret_cast<const uint4*>(p); }

template <typename Tin, typename Tr, int D, bool MASKED>
__global__ __launch_bounds__(kPoolThreads) void pool_tile_kernel(
    const Tin* __restrict__ child, int64_t in_unit_stride, const Tr* __restrict__ Rall,
    PoolOut out, int nlev, int Hkv, int tile_begin, int tile_end, int row_limit, int b,
    float tau) {
  constexpr bool kBF = sizeof(Tin) == 2;
  constexpr int RWb = D / 2 + 4;  // bf16 row stride in dwords (padding spreads banks)
  constexpr int RWf = D + 4;      // fp32 row stride in floats
  constexpr int IN_WORDS = kBF ? kTileRows * RWb : kTileRows * RWf;
  __shared__ uint32_t sIn[IN_WORDS];
  __shared__ float sY[2][(kTileRows / 2) * RWf];
  __shared__ float zs[kTileRows][kNRef + 1];
  __shared__ float sw[kTileRows];

  const int unit = blockIdx.y;
  const int g = unit % Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mem = lane & 15, grp = lane >> 4;
  int TR = 1;
  for (int j = 0; j < nlev; ++j) TR *= b;

  // B operands: R^T. bf16 form for bf16 children, float32 form for float32 levels.
  const Tr* R = Rall + (int64_t)g * kNRef * D;
  bf16x8_t rb[D / 32];
  float rf[D / 16][4];
#pragma unroll
  for (int kc = 0; kc < D / 32; ++kc) {
    if constexpr (kBF)
      rb[kc] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(R + mem * D + 32 * kc + 8 * grp));
    else
      rb[kc] = bf16x8_t{};
  }
#pragma unroll
  for (int q = 0; q < D / 16; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) rf[q][e] = to_f32(R[mem * D + 16 * q + 4 * grp + e]);

  // child rows of tile t go through registers: the next tile's loads are issued before
  // the current tile is pooled
  constexpr int VPR = kBF ? D / 8 : D / 4;   // 16-byte vectors per row
  constexpr int PRE = kTileRows * VPR / kPoolThreads;
  u32x4_t pre[PRE];
  const u32x4_t* tiles = reinterpret_cast<const u32x4_t*>(child + unit * in_unit_stride);
  const int tvec = TR * VPR;  // 16-byte vectors per tile
  const int tfirst = tile_begin + blockIdx.x * kTilesPerWG;
  if (tfirst < tile_end) {
#pragma unroll
    for (int q = 0; q < PRE; ++q) {
      const int i = min((int)threadIdx.x + q * kPoolThreads, tvec - 1);
      pre[q] = tiles[(int64_t)tfirst * tvec + i];
    }
  }
  for (int ti = 0; ti < kTilesPerWG; ++ti) {
    const int t = tfirst + ti;
    if (t >= tile_end) break;
    __syncthreads();  // the previous tile is fully consumed
#pragma unroll
    for (int q = 0; q < PRE; ++q) {
      const int i = threadIdx.x + q * kPoolThreads;
      if (i < TR * VPR) {
        const int r = i / VPR, c = i % VPR;
        *reinterpret_cast<u32x4_t*>(&sIn[r * (kBF ? RWb : RWf) + 4 * c]) = pre[q];
      }
    }
    __syncthreads();
    if (ti + 1 < kTilesPerWG && t + 1 < tile_end) {
#pragma unroll
      for (int q = 0; q < PRE; ++q) {
        const int i = min((int)threadIdx.x + q * kPoolThreads, tvec - 1);
        pre[q] = tiles[(int64_t)(t + 1) * tvec + i];
      }
    }

    int rows = TR;
    // child rows at or past row_limit are not cached yet: only nodes whose children are all
    // valid are stored (the others only feed nodes that are not stored either)
    int vrows = MASKED ? min(TR, row_limit - t * TR) : TR;
    for (int j = 0; j < nlev; ++j) {
      const bool bf_in = kBF && j == 0;
      const float* inF = (j == 0) ? reinterpret_cast<const float*>(sIn) : sY[(j - 1) & 1];
      // z^T for this level's rows, 16 rows per MFMA block, one block per wave
      for (int blk = wave; blk * 16 < rows; blk += kPoolThreads / 64) {
        const int row = 16 * blk + mem;
        const bool rv = row < rows;
        f32x4_t zc = {0.f, 0.f, 0.f, 0.f};
        if (bf_in) {
#pragma unroll
          for (int kc = 0; kc < D / 32; ++kc) {
            const uint4 a = rv ? lds16(&sIn[row * RWb + 16 * kc + 4 * grp]) : make_uint4(0u, 0u, 0u, 0u);
            zc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), rb[kc], zc,
                                                         0, 0, 0);
          }
        } else {
#pragma unroll
          for (int q = 0; q < D / 16; ++q) {
            const float4 a = rv ? *reinterpret_cast<const float4*>(&inF[row * RWf + 16 * q + 4 * grp])
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            zc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, rf[q][0], zc, 0, 0, 0);
            zc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, rf[q][1], zc, 0, 0, 0);
            zc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, rf[q][2], zc, 0, 0, 0);
            zc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, rf[q][3], zc, 0, 0, 0);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int zr = 16 * blk + 4 * grp + r;
          if (zr < rows) zs[zr][mem] = tau * zc[r];
        }
      }
      __syncthreads();
      const int nodes = rows / b;
      // softmax over each node's children, per reference query
      for (int i = threadIdx.x; i < nodes * kNRef; i += kPoolThreads) {
        const int nd = i / kNRef, rf_ = i % kNRef;
        float mx = -INFINITY;
        for (int c = 0; c < b; ++c) mx = fmaxf(mx, zs[nd * b + c][rf_]);
        float sum = 0.f;
        for (int c = 0; c < b; ++c) sum += expf(zs[nd * b + c][rf_] - mx);
        for (int c = 0; c < b; ++c) zs[nd * b + c][rf_] = expf(zs[nd * b + c][rf_] - mx) / sum;
      }
      __syncthreads();
      for (int r = threadIdx.x; r < rows; r += kPoolThreads) {
        float s = 0.f;
#pragma unroll
        for (int rf_ = 0; rf_ < kNRef; ++rf_) s += zs[r][rf_];
        sw[r] = s * (1.f / kNRef);
      }
      __syncthreads();
      float* dst = out.ptr[j] + unit * out.unit_stride[j] + (int64_t)t * nodes * D;
      float* ynext = sY[j & 1];
      const int vnodes = vrows / b;
      for (int i = threadIdx.x; i < nodes * D; i += kPoolThreads) {
        const int nd = i / D, k = i % D;
        float acc = 0.f;
        for (int c = 0; c < b; ++c) {
          const int r = nd * b + c;
          float x;
          if (bf_in) {
            const uint32_t w = sIn[r * RWb + (k >> 1)];
            x = __uint_as_float((k & 1) ? (w & 0xffff0000u) : (w << 16));
          } else {
            x = inF[r * RWf + k];
          }
          acc = fmaf(sw[r], x, acc);
        }
        if (nd < vnodes) dst[(int64_t)nd * D + k] = acc;
        if (j + 1 < nlev) ynext[nd * RWf + k] = acc;
      }
      __syncthreads();
      rows = nodes;
      vrows = vnodes;
    }
  }
}

// ------------------------------------------------------------------------------------
// Deep trees (b = 4) over bf16 keys: wave-centric fused pooling of up to three levels.
// Each wave owns 64 consecutive key rows (16 level-1 nodes, 4 level-2 nodes, 1 level-3
// node) and pools them with no workgroup barrier:
//  * z^T = K . R^T on v_mfma_f32_16x16x32_bf16 with the 16-row block loaded straight into
//    A-operand registers; the C layout gives lane (ref = l % 16, group g = l / 16) the
//    scores of rows 4g..4g+3, i.e. of all four children of node g, so the softmax over
//    children is lane-local; the mean over references is a 16-lane reduction;
//  * the rows go through a small per-wave LDS tile, and lane l sums the four children of
//    node l / 16 over dims 8 (l % 16) .. +8 (its weights are already in its lane group);
//  * levels 2 and 3 repeat this on the float32 rows kept in LDS (v_mfma_f32_16x16x4_f32).
// The arithmetic for a node never depends on its position, so identical subtrees give
// identical summaries.
constexpr int kWaveRows = 64;
constexpr int kWaveTilesPerWave = 2;

// MXFP4 encoding of a row the wave kernel just pooled, where each of 16 lanes (one lane
// group) holds DL = D / 16 consecutive elements: the lanes of a 32-element block agree on
// its largest magnitude by shuffles, each writes its DL codes, the block's first lane the
// scale. The values are the float32 results stored to the pyramid, so the codes equal
// those the standalone encoder writes from the stored rows.
template <int D>
__device__ __forceinline__ void wave_encode_row(const float* acc, int mem, bool store,
                                                uint8_t* codes_row, uint8_t* scales_row) {
  constexpr int DL = D / 16;
  constexpr int LPB = kMxBlock / DL;  // lanes per block
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < DL; ++i) amax = fmaxf(amax, fabsf(acc[i]));
#pragma unroll
  for (int off = 1; off < LPB; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const uint32_t sb = mx_scale_byte(amax);
  const float inv = mx_inv_scale(sb);
  const uint32_t w = e2m1_pack(acc, DL, inv);
  if (store) {
    if constexpr (DL == 8)
      reinterpret_cast<uint32_t*>(codes_row)[mem] = w;
    else
      reinterpret_cast<uint16_t*>(codes_row)[mem] = (uint16_t)w;
    if (mem % LPB == 0) scales_row[mem / LPB] = (uint8_t)sb;
  }
}

template <int D, bool MASKED, bool ENC>
__global__ __launch_bounds__(kPoolThreads, ENC ? 2 : 3) void pool_wave_b4_kernel(
    const bf16_t* __restrict__ child, int64_t in_unit_stride, const bf16_t* __restrict__ Rall,
    PoolOut out, int nlev, int Hkv, int tile_begin, int tile_end, int row_limit, float tau) {
  constexpr int KC = D / 32;
  constexpr int NQ = D / 16;
  constexpr int RWb = D / 2 + 4;  // bf16 raw-row stride in dwords
  constexpr int RWf = D + 4;      // float row stride
  constexpr int DL = D / 16;      // output dims per lane in the weighted sums
  // the level-2 rows (levels 2 -> 3) reuse the raw-row tile, free once level 1 is done:
  // 51 KB per workgroup at d = 128, so three workgroups fit in a CU's LDS
  static_assert(4 * RWf <= 16 * RWb, "level-2 rows must fit in the raw-row tile");
  __shared__ uint32_t sRaw[4][16 * RWb];
  __shared__ float sL1[4][16 * RWf];

  const int unit = blockIdx.y;
  const int g_kv = unit % Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mem = lane & 15, grp = lane >> 4;

  const bf16_t* R = Rall + (int64_t)g_kv * kNRef * D;
  bf16x8_t rb[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    rb[kc] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(R + mem * D + 32 * kc + 8 * grp));
  float rf[NQ][4];
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) rf[q][e] = to_f32(R[mem * D + 16 * q + 4 * grp + e]);

  uint32_t* raw = sRaw[wave];
  float* l1 = sL1[wave];
  float* l2 = reinterpret_cast<float*>(sRaw[wave]);

  // child weights of node `grp` from this lane's four scores z[r] (rows 4 grp + r):
  // softmax over the children, then the mean over the 16 references of the lane group
  auto weights = [&](const f32x4_t& zc, float w[4]) {
    float z[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) z[r] = tau * zc[r];
    const float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    float e[4], sum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      e[r] = expf(z[r] - mx);
      sum += e[r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float a = e[r] / sum;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) a += __shfl_xor(a, off, 64);
      w[r] = a * (1.f / kNRef);
    }
  };

  for (int it = 0; it < kWaveTilesPerWave; ++it) {
    const int t = tile_begin + (blockIdx.x * (kPoolThreads / 64) + wave) * kWaveTilesPerWave + it;
    if (t >= tile_end) break;
    const bf16_t* src = child + unit * in_unit_stride + (int64_t)t * kWaveRows * D;
    // rows at or past row_limit are not cached yet: only complete nodes are stored
    const int vrows = MASKED ? min(kWaveRows, row_limit - t * kWaveRows) : kWaveRows;
    uint4 a[4][KC];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        a[blk][kc] = *reinterpret_cast<const uint4*>(src + (int64_t)(16 * blk + mem) * D + 32 * kc + 8 * grp);

    // level 1: four 16-row blocks -> 16 nodes
    float* dst1 = out.ptr[0] + unit * out.unit_stride[0] + (int64_t)t * 16 * D;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      f32x4_t zc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        zc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[blk][kc]), rb[kc], zc,
                                                     0, 0, 0);
      float w[4];
      weights(zc, w);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        *reinterpret_cast<uint4*>(&raw[mem * RWb + 16 * kc + 4 * grp]) = a[blk][kc];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // node grp of this block, dims DL * mem .. + DL
      float acc[DL];
#pragma unroll
      for (int i = 0; i < DL; ++i) acc[i] = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t* rp = &raw[(4 * grp + c) * RWb + (DL / 2) * mem];
#pragma unroll
        for (int i = 0; i < DL / 2; ++i) {
          const uint32_t v = rp[i];
          acc[2 * i] = fmaf(w[c], __uint_as_float(v << 16), acc[2 * i]);
          acc[2 * i + 1] = fmaf(w[c], __uint_as_float(v & 0xffff0000u), acc[2 * i + 1]);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int node = 4 * blk + grp;
      const bool st1 = 4 * (node + 1) <= vrows;
#pragma unroll
      for (int i = 0; i < DL; i += 4) {
        const float4 o = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
        if (st1) *reinterpret_cast<float4*>(dst1 + (int64_t)node * D + DL * mem + i) = o;
        *reinterpret_cast<float4*>(&l1[node * RWf + DL * mem + i]) = o;
      }
      if constexpr (ENC) {
        const int64_t row = unit * (out.unit_stride[0] / D) + (int64_t)t * 16 + node;
        wave_encode_row<D>(acc, mem, st1, out.codes[0] + row * (D / 2),
                           out.scales[0] + row * (D / kMxBlock));
      }
    }
    if (nlev < 2) continue;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // levels 2 and 3 from the float32 rows in LDS (16 rows, then 4)
    for (int j = 1; j < nlev; ++j) {
      const float* in = (j == 1) ? l1 : l2;
      const int rows = (j == 1) ? 16 : 4;
      f32x4_t zc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const float4 x = mem < rows ? *reinterpret_cast<const float4*>(&in[mem * RWf + 16 * q + 4 * grp])
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
        zc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.x, rf[q][0], zc, 0, 0, 0);
        zc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.y, rf[q][1], zc, 0, 0, 0);
        zc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.z, rf[q][2], zc, 0, 0, 0);
        zc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.w, rf[q][3], zc, 0, 0, 0);
      }
      float w[4];
      weights(zc, w);
      const int nodes = rows / 4;
      if (grp < nodes) {
        float acc[DL];
#pragma unroll
        for (int i = 0; i < DL; ++i) acc[i] = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float* rp = &in[(4 * grp + c) * RWf + DL * mem];
#pragma unroll
          for (int i = 0; i < DL; ++i) acc[i] = fmaf(w[c], rp[i], acc[i]);
        }
        float* dst = out.ptr[j] + unit * out.unit_stride[j] + ((int64_t)t * nodes + grp) * D;
        const int span = j == 1 ? 16 : 64;  // key rows under one node of this level
        const bool stj = span * (grp + 1) <= vrows;
#pragma unroll
        for (int i = 0; i < DL; i += 4) {
          const float4 o = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
          if (stj) *reinterpret_cast<float4*>(dst + DL * mem + i) = o;
          if (j == 1) *reinterpret_cast<float4*>(&l2[grp * RWf + DL * mem + i]) = o;
        }
        if constexpr (ENC) {
          const int64_t row = unit * (out.unit_stride[j] / D) + (int64_t)t * nodes + grp;
          wave_encode_row<D>(acc, mem, stj, out.codes[j] + row * (D / 2),
                             out.scales[j] + row * (D / kMxBlock));
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

// ------------------------------------------------------------------------------------
// Upper levels of deep trees (b = 4): the same wave-centric pooling of three levels over
// float32 child rows (a stored pyramid level). Each wave owns 64 consecutive child rows;
// a 16-row block at a time is loaded into A-operand registers, scored on
// v_mfma_f32_16x16x4_f32 (the C layout again gives each lane all four children of one
// node for one reference), staged in the wave's LDS tile for the weighted sums, and the
// two levels above repeat this on the rows kept in LDS. No workgroup barrier; a node's
// arithmetic never depends on its position.
template <typename Tr, int D, bool MASKED>
__global__ __launch_bounds__(kPoolThreads) void pool_wave_f32_kernel(
    const float* __restrict__ child, int64_t in_unit_stride, const Tr* __restrict__ Rall,
    PoolOut out, int nlev, int Hkv, int tile_begin, int tile_end, int row_limit, float tau) {
  constexpr int NQ = D / 16;
  constexpr int RWf = D + 4;  // float row stride (padding spreads banks)
  constexpr int DL = D / 16;  // output dims per lane in the weighted sums
  __shared__ float sRaw[4][16 * RWf];  // a block's child rows; later the middle level's rows
  __shared__ float sL1[4][16 * RWf];   // the first pooled level's 16 rows

  const int unit = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mem = lane & 15, grp = lane >> 4;
  const int t = tile_begin + blockIdx.x * (kPoolThreads / 64) + wave;
  if (t >= tile_end) return;

  const Tr* R = Rall + (int64_t)(unit % Hkv) * kNRef * D;
  float rf[NQ][4];
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) rf[q][e] = to_f32(R[mem * D + 16 * q + 4 * grp + e]);
  float* raw = sRaw[wave];
  float* l1 = sL1[wave];

  auto weights = [&](const f32x4_t& zc, float w[4]) {
    float z[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) z[r] = tau * zc[r];
    const float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    float e[4], sum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      e[r] = expf(z[r] - mx);
      sum += e[r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float a = e[r] / sum;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) a += __shfl_xor(a, off, 64);
      w[r] = a * (1.f / kNRef);
    }
  };
  auto score = [&](const f32x4_t (&x)[NQ]) {
    f32x4_t zc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      zc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[q][0], rf[q][0], zc, 0, 0, 0);
      zc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[q][1], rf[q][1], zc, 0, 0, 0);
      zc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[q][2], rf[q][2], zc, 0, 0, 0);
      zc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[q][3], rf[q][3], zc, 0, 0, 0);
    }
    return zc;
  };
  // lane (mem, grp): node grp's weighted sum over dims DL mem .. + DL from rows `in`
  auto pooled = [&](const float* in, const float w[4], float (&acc)[DL]) {
#pragma unroll
    for (int i = 0; i < DL; ++i) acc[i] = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float* rp = &in[(4 * grp + c) * RWf + DL * mem];
#pragma unroll
      for (int i = 0; i < DL; ++i) acc[i] = fmaf(w[c], rp[i], acc[i]);
    }
  };

  const float* src = child + unit * in_unit_stride + (int64_t)t * kWaveRows * D;
  // child rows at or past row_limit are not cached yet: only complete nodes are stored
  const int vrows = MASKED ? min(kWaveRows, row_limit - t * kWaveRows) : kWaveRows;
  float* dst1 = out.ptr[0] + unit * out.unit_stride[0] + (int64_t)t * 16 * D;
  f32x4_t x[NQ], xn[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q)
    x[q] = *reinterpret_cast<const f32x4_t*>(src + (int64_t)mem * D + 16 * q + 4 * grp);
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    if (blk + 1 < 4) {  // the next block's rows are in flight while this one is pooled
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        xn[q] = *reinterpret_cast<const f32x4_t*>(src + (int64_t)(16 * (blk + 1) + mem) * D +
                                                  16 * q + 4 * grp);
    }
    float w[4];
    weights(score(x), w);
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      *reinterpret_cast<f32x4_t*>(&raw[mem * RWf + 16 * q + 4 * grp]) = x[q];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float acc[DL];
    pooled(raw, w, acc);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int node = 4 * blk + grp;
    const bool st1 = 4 * (node + 1) <= vrows;
#pragma unroll
    for (int i = 0; i < DL; i += 4) {
      const float4 o = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
      if (st1) *reinterpret_cast<float4*>(dst1 + (int64_t)node * D + DL * mem + i) = o;
      *reinterpret_cast<float4*>(&l1[node * RWf + DL * mem + i]) = o;
    }
    if (blk + 1 < 4) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) x[q] = xn[q];
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // the two levels above, from the rows in LDS (16 rows, then 4 kept in the raw tile)
  for (int j = 1; j < nlev; ++j) {
    const float* in = (j == 1) ? l1 : raw;
    const int rows = (j == 1) ? 16 : 4;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      x[q] = mem < rows ? *reinterpret_cast<const f32x4_t*>(&in[mem * RWf + 16 * q + 4 * grp])
                        : f32x4_t{0.f, 0.f, 0.f, 0.f};
    float w[4];
    weights(score(x), w);
    const int nodes = rows / 4;
    if (grp < nodes) {
      float acc[DL];
      pooled(in, w, acc);
      float* dst = out.ptr[j] + unit * out.unit_stride[j] + ((int64_t)t * nodes + grp) * D;
      const int span = j == 1 ? 16 : 64;  // child rows under one node of this level
      const bool stj = span * (grp + 1) <= vrows;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int i = 0; i < DL; i += 4) {
        const float4 o = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
        if (stj) *reinterpret_cast<float4*>(dst + DL * mem + i) = o;
        if (j == 1) *reinterpret_cast<float4*>(&raw[grp * RWf + DL * mem + i]) = o;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// ------------------------------------------------------------------------------------
// Wide nodes (64 < b <= 256) over bf16 keys: one workgroup per node, wave w owns children
// 64 w .. 64 w + 63, loaded straight into the A operand of v_mfma_f32_16x16x32_bf16
// (z = tau R x^T, 16 children x 16 references per block). Each reference's softmax max
// and normaliser over all b children combine across the four waves through LDS; each
// child's weight (mean over references) is formed on the MFMA C layout, moved to the
// A-layout lanes by shuffles, and the weighted sum of the wave's children is reduced
// across lanes and then across waves in a fixed order.
constexpr int kWideNodeMax = 256;

template <int D>
__global__ __launch_bounds__(kPoolThreads) void pool_wide_kernel(
    const bf16_t* __restrict__ child, int64_t in_unit_stride, const bf16_t* __restrict__ Rall,
    float* __restrict__ out, int64_t out_unit_stride, int Hkv, int node_begin, int node_end,
    int b, float tau) {
  constexpr int KC = D / 32;
  constexpr int NW = kPoolThreads / 64;
  __shared__ float sMax[NW][kNRef], sSum[NW][kNRef];
  __shared__ float sPart[NW][D];
  const int unit = blockIdx.y;
  const int node = node_begin + blockIdx.x;
  if (node >= node_end) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mem = lane & 15, grp = lane >> 4;
  const bf16_t* R = Rall + (int64_t)(unit % Hkv) * kNRef * D;
  bf16x8_t rb[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    rb[kc] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(R + mem * D + 32 * kc + 8 * grp));

  // child rows c = 64 wave + 16 blk + mem (rows at or past b: row 0, masked)
  const bf16_t* base = child + unit * in_unit_stride + (int64_t)node * b * D;
  uint4 a[4][KC];
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    const int c = 64 * wave + 16 * blk + mem;
    const bf16_t* row = base + (int64_t)(c < b ? c : 0) * D + 8 * grp;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) a[blk][kc] = *reinterpret_cast<const uint4*>(row + 32 * kc);
  }
  // z for rows 16 blk + 4 grp + r and reference `mem`
  float z[4][4];
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    f32x4_t zc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      zc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[blk][kc]),
                                                   rb[kc], zc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = 64 * wave + 16 * blk + 4 * grp + r;
      z[blk][r] = c < b ? tau * zc[r] : -INFINITY;
    }
  }
  // per-reference max and normaliser over all children
  float m = -INFINITY;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk)
#pragma unroll
    for (int r = 0; r < 4; ++r) m = fmaxf(m, z[blk][r]);
  m = fmaxf(m, __shfl_xor(m, 16, 64));
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  if (grp == 0) sMax[wave][mem] = m;
  __syncthreads();
  float M = sMax[0][mem];
#pragma unroll
  for (int v = 1; v < NW; ++v) M = fmaxf(M, sMax[v][mem]);
  float e[4][4], ssum = 0.f;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      e[blk][r] = expf(z[blk][r] - M);
      ssum += e[blk][r];
    }
  ssum += __shfl_xor(ssum, 16, 64);
  ssum += __shfl_xor(ssum, 32, 64);
  if (grp == 0) sSum[wave][mem] = ssum;
  __syncthreads();
  float S = 0.f;
#pragma unroll
  for (int v = 0; v < NW; ++v) S += sSum[v][mem];
  // weight of rows 16 blk + 4 grp + r: mean over the 16 references (lanes mem = 0..15)
  float w[4][4];
#pragma unroll
  for (int blk = 0; blk < 4; ++blk)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float t = e[blk][r] / S;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) t += __shfl_xor(t, off, 64);
      w[blk][r] = t * (1.f / kNRef);
    }
  // this lane's A row is 16 blk + mem: its weight sits in lanes of group mem / 4, entry
  // mem % 4
  float acc[KC][8];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[kc][i] = 0.f;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    const int src = 16 * (mem >> 2);
    const float w0 = __shfl(w[blk][0], src, 64), w1 = __shfl(w[blk][1], src, 64);
    const float w2 = __shfl(w[blk][2], src, 64), w3 = __shfl(w[blk][3], src, 64);
    const int rsel = mem & 3;
    const float wr = rsel == 0 ? w0 : (rsel == 1 ? w1 : (rsel == 2 ? w2 : w3));
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const uint4 v = a[blk][kc];
      const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[kc][2 * i] = fmaf(wr, __uint_as_float(wd[i] << 16), acc[kc][2 * i]);
        acc[kc][2 * i + 1] = fmaf(wr, __uint_as_float(wd[i] & 0xffff0000u), acc[kc][2 * i + 1]);
      }
    }
  }
  // sum over the 16 rows (lanes mem = 0..15) of each group: dims 32 kc + 8 grp + i
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float t = acc[kc][i];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) t += __shfl_xor(t, off, 64);
      acc[kc][i] = t;
    }
  if (mem == 0) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int i = 0; i < 8; ++i) sPart[wave][32 * kc + 8 * grp + i] = acc[kc][i];
  }
  __syncthreads();
  for (int k = threadIdx.x; k < D; k += kPoolThreads) {
    float t = sPart[0][k];
#pragma unroll
    for (int v = 1; v < NW; ++v) t += sPart[v][k];
    out[unit * out_unit_stride + (int64_t)node * D + k] = t;
  }
}

template <int D>
hipError_t launch_wave_b4(const void* child, int64_t in_unit_stride, const void* R,
                          const PoolOut& out, int nlev, int units, int Hkv, int row_begin,
                          int row_end, int row_limit, hipStream_t s) {
  const int t0 = row_begin / kWaveRows, t1 = row_end / kWaveRows;
  if (t1 <= t0) return hipSuccess;
  const int per_wg = (kPoolThreads / 64) * kWaveTilesPerWave;
  dim3 grid((t1 - t0 + per_wg - 1) / per_wg, units);
  // tiles that all lie below row_limit store every node: the unmasked form
  const float tau = 1.0f / sqrtf((float)D);
#define ZHA_WAVE(M, E)                                                                        \
  hipLaunchKernelGGL((pool_wave_b4_kernel<D, M, E>), grid, dim3(kPoolThreads), 0, s,           \
                     (const bf16_t*)child, in_unit_stride, (const bf16_t*)R, out, nlev, Hkv, t0, \
                     t1, row_limit, tau)
  const bool masked = row_limit < row_end, enc = out.codes[0] != nullptr;
  if (!masked && !enc) ZHA_WAVE(false, false);
  else if (!masked) ZHA_WAVE(false, true);
  else if (!enc) ZHA_WAVE(true, false);
  else ZHA_WAVE(true, true);
#undef ZHA_WAVE
  return hipGetLastError();
}

template <typename Tr, int D>
hipError_t launch_wave_f32(const void* child, int64_t in_unit_stride, const void* R,
                           const PoolOut& out, int nlev, int units, int Hkv, int row_begin,
                           int row_end, int row_limit, hipStream_t s) {
  const int t0 = row_begin / kWaveRows, t1 = row_end / kWaveRows;
  if (t1 <= t0) return hipSuccess;
  const int per_wg = kPoolThreads / 64;  // one tile per wave
  dim3 grid((t1 - t0 + per_wg - 1) / per_wg, units);
  const float tau = 1.0f / sqrtf((float)D);
  if (row_limit < row_end)
    hipLaunchKernelGGL((pool_wave_f32_kernel<Tr, D, true>), grid, dim3(kPoolThreads), 0, s,
                       (const float*)child, in_unit_stride, (const Tr*)R, out, nlev, Hkv, t0, t1,
                       row_limit, tau);
  else
    hipLaunchKernelGGL((pool_wave_f32_kernel<Tr, D, false>), grid, dim3(kPoolThreads), 0, s,
                       (const float*)child, in_unit_stride, (const Tr*)R, out, nlev, Hkv, t0, t1,
                       row_limit, tau);
  return hipGetLastError();
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
  } else if (sizeof(Tin) == 2 && sizeof(Tr) == 2 && b <= kWideNodeMax) {
    // bf16 keys: the wave-centric wide-node kernel
    dim3 grid(nodes, units);
    hipLaunchKernelGGL((pool_wide_kernel<D>), grid, dim3(kPoolThreads), 0, s,
                       (const bf16_t*)child, in_unit_stride, (const bf16_t*)R, out,
                       out_unit_stride, Hkv, node_begin, node_end, b, tau);
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

template <typename Tin, typename Tr, int D>
hipError_t launch_tile_t(const void* child, int64_t in_unit_stride, const void* R,
                         const PoolOut& out, int nlev, int units, int Hkv, int row_begin,
                         int row_end, int row_limit, int b, hipStream_t s) {
  int TR = 1;
  for (int j = 0; j < nlev; ++j) TR *= b;
  const int t0 = row_begin / TR, t1 = row_end / TR;
  if (t1 <= t0) return hipSuccess;
  dim3 grid((t1 - t0 + kTilesPerWG - 1) / kTilesPerWG, units);
  if (row_limit >= row_end)
    hipLaunchKernelGGL((pool_tile_kernel<Tin, Tr, D, false>), grid, dim3(kPoolThreads), 0, s,
                       (const Tin*)child, in_unit_stride, (const Tr*)R, out, nlev, Hkv, t0, t1,
                       row_limit, b, 1.0f / sqrtf((float)D));
  else
    hipLaunchKernelGGL((pool_tile_kernel<Tin, Tr, D, true>), grid, dim3(kPoolThreads), 0, s,
                       (const Tin*)child, in_unit_stride, (const Tr*)R, out, nlev, Hkv, t0, t1,
                       row_limit, b, 1.0f / sqrtf((float)D));
  return hipGetLastError();
}

template <typename Tin, typename Tr>
hipError_t launch_tile_d(int D, const void* child, int64_t in_unit_stride, const void* R,
                         const PoolOut& out, int nlev, int units, int Hkv, int row_begin,
                         int row_end, int row_limit, int b, hipStream_t s) {
  if (D == 64)
    return launch_tile_t<Tin, Tr, 64>(child, in_unit_stride, R, out, nlev, units, Hkv,
                                      row_begin, row_end, row_limit, b, s);
  return launch_tile_t<Tin, Tr, 128>(child, in_unit_stride, R, out, nlev, units, Hkv, row_begin,
                                     row_end, row_limit, b, s);
}

}  // namespace

int fused_levels(int b, int levels_left) {
  int k = 0, tr = 1;
  while (k < levels_left && k < kMaxFuse && tr * b <= kTileRows) {
    tr *= b;
    ++k;
  }
  return k;
}

bool pool_fused_encodes(int dtype_in, int dtype_r, int b, int nlev, int row_begin,
                        int row_end) {
  return dtype_r == ZHA_BF16 && dtype_in == ZHA_BF16 && b == 4 && nlev <= 3 &&
         row_begin % kWaveRows == 0 && row_end % kWaveRows == 0;
}

hipError_t launch_pool_fused(int dtype_in, const void* child, int64_t in_unit_stride,
                             const void* R, int dtype_r, float* const* outs,
                             const int64_t* out_unit_strides, int nlev, int units, int Hkv,
                             int row_begin, int row_end, int row_limit, int b, int D,
                             uint8_t* const* rcodes, uint8_t* const* rscales, hipStream_t s) {
  if (nlev < 1 || nlev > kMaxFuse) return hipErrorInvalidValue;
  PoolOut out{};
  for (int j = 0; j < nlev; ++j) {
    out.ptr[j] = outs[j];
    out.unit_stride[j] = out_unit_strides[j];
    out.codes[j] = rcodes ? rcodes[j] : nullptr;
    out.scales[j] = rscales ? rscales[j] : nullptr;
  }
  if (dtype_in == ZHA_F32 && b == 4 && nlev == 3 && !out.codes[0]) {
    // three upper levels of a deep tree over a stored float32 level: 64-row tiles (every
    // launch of these levels is whole tiles, so each node always takes this kernel)
    if (dtype_r == ZHA_BF16)
      return D == 64 ? launch_wave_f32<bf16_t, 64>(child, in_unit_stride, R, out, nlev, units,
                                                   Hkv, row_begin, row_end, row_limit, s)
                     : launch_wave_f32<bf16_t, 128>(child, in_unit_stride, R, out, nlev, units,
                                                    Hkv, row_begin, row_end, row_limit, s);
    return D == 64 ? launch_wave_f32<float, 64>(child, in_unit_stride, R, out, nlev, units, Hkv,
                                                row_begin, row_end, row_limit, s)
                   : launch_wave_f32<float, 128>(child, in_unit_stride, R, out, nlev, units, Hkv,
                                                 row_begin, row_end, row_limit, s);
  }
  if (dtype_r == ZHA_BF16) {
    // bf16 keys, b = 4, rows in whole 64-row wave tiles: the wave-centric kernel (the
    // only one that also writes the router copy)
    if (pool_fused_encodes(dtype_in, dtype_r, b, nlev, row_begin, row_end)) {
      if (D == 64)
        return launch_wave_b4<64>(child, in_unit_stride, R, out, nlev, units, Hkv, row_begin,
                                  row_end, row_limit, s);
      return launch_wave_b4<128>(child, in_unit_stride, R, out, nlev, units, Hkv, row_begin,
                                 row_end, row_limit, s);
    }
    if (dtype_in == ZHA_BF16)
      return launch_tile_d<bf16_t, bf16_t>(D, child, in_unit_stride, R, out, nlev, units, Hkv,
                                           row_begin, row_end, row_limit, b, s);
    return launch_tile_d<float, bf16_t>(D, child, in_unit_stride, R, out, nlev, units, Hkv,
                                        row_begin, row_end, row_limit, b, s);
  }
  return launch_tile_d<float, float>(D, child, in_unit_stride, R, out, nlev, units, Hkv,
                                     row_begin, row_end, row_limit, b, s);
}

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
