// Sparse attention over the top-k selected positions (gfx950).
//
// DSA glossary entry ("Optimizing speculative decoding", section "IndexShare
// and KVShare"): full attention runs over only the selected subset.  With
// IndexShare every draft step passes the same index set, so each step reads
// only target-written KV.
//
// Per-head KV (H_q / H_kv in {1, 2, 4}, D in {64, 128}): the work is a gather
// of k KV rows per head with one FMA per byte, so it is HBM-bound and runs on
// VALU, not MFMA.  A KV row of D bf16 is read by D/8 lanes (16 bytes each);
// a wave covers 64/(D/8) KV heads of one token, so every load instruction
// reads one contiguous stretch of the token's K (or V) row.  The workgroup's
// waves walk disjoint tokens of its split with their own online-softmax
// state (exp2 domain), merge in LDS in a fixed order, and write either the
// final output (one split) or a partial (o, m, l) that a combine kernel folds
// in split order.
//
// Latent MQA (H_kv = 1, D_qk = 576, D_v = 512): every query head reads the
// same gathered rows, so QK^T and PV are dense contractions over the heads and
// run on bf16 MFMA (see latent_attn_kernel).
#include <cmath>
#include <mutex>

#include "dsa_common.h"

namespace dsa {
namespace {

#ifndef DSA_ATTN_WAVES
#define DSA_ATTN_WAVES 8
#endif
constexpr int kWaves = DSA_ATTN_WAVES;      // waves per per-head-KV workgroup
constexpr int kThreads = kWaves * 64;
// A streamed gather (one query row per sequence, larger than the last-level
// cache) with one query head per KV head runs 16 waves per workgroup, so one
// workgroup holds all k = 2048 tokens of a (sequence, head group) and the
// call needs no split-k combine launch (8 waves: 2 splits plus the combine).
#ifndef DSA_ATTN_STREAM_WAVES
#define DSA_ATTN_STREAM_WAVES 16
#endif
constexpr int kStreamWaves = DSA_ATTN_STREAM_WAVES;

// Split-k plan: aim for about kTargetGroups workgroups, each with at least
// kMinTokens selected tokens (tunable at build time).
#ifndef DSA_ATTN_TARGET_WGS
#define DSA_ATTN_TARGET_WGS 1024
#endif
#ifndef DSA_ATTN_TARGET_WGS_STREAM
#define DSA_ATTN_TARGET_WGS_STREAM 256
#endif
#ifndef DSA_ATTN_MIN_TOKENS
#define DSA_ATTN_MIN_TOKENS 256
#endif
#ifndef DSA_ATTN_UNROLL
#define DSA_ATTN_UNROLL 2
#endif
#ifndef DSA_ATTN_UNROLL_NT
#define DSA_ATTN_UNROLL_NT 4
#endif

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  int64_t page_stride, row_stride, head_stride;
  const int32_t* bt;
  const int32_t* idx;
  int idx_rows;
  int S_q, H_q, H_kv, page, max_pages, k;
  float scale_log2;        // sm_scale * log2(e)
  float* out;
  float* lse;
  float* part_o;           // [B*S_q*H_q][nsplit][D_v]
  float* part_ml;          // [B*S_q*H_q][nsplit][2]
  int batch, head_groups;
  int row_grouped;         // 1: flat grid, the S_q rows of one (b, split, head group) share an XCD
  int nsplit;
  int tok_per_split;
};

constexpr int kMaxTokPerSplit = 1024;
#ifndef DSA_ATTN_STREAM_BYTES
#define DSA_ATTN_STREAM_BYTES (256ll << 20)
#endif
constexpr long long kAttnStreamBytes = DSA_ATTN_STREAM_BYTES;   // last-level cache (MALL) size

// ---------------------------------------------------------------------------
// Per-head KV gather kernel
// ---------------------------------------------------------------------------
// Row offsets (elements) of a wave's tokens: lane l holds those of the
// wave's local tokens l and l + 64 (-1: absent).  A token's offset is the
// same for the whole wave, so it is read into scalar registers (readlane)
// and each K/V load adds the lane's 32-bit byte offset inside the row.
struct WaveRows {
  int64_t o0, o1;
  int nw;          // tokens of this wave
};
static_assert(kMaxTokPerSplit <= 128 * kWaves, "a wave's tokens fit in two offsets per lane");
constexpr int kStreamTokPerSplit = 128 * kStreamWaves;   // tokens per split of the 16-wave streamed gather

__device__ __forceinline__ int64_t row_off(const WaveRows& r, int j) {   // j wave-uniform
  const int jj = min(j, max(r.nw - 1, 0));
  const int64_t v = jj < 64 ? r.o0 : r.o1;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, jj & 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), jj & 63);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// 16 bytes of a KV row; NT: non-temporal (a gather far larger than the
// last-level cache, whose rows are not read again by this call)
template <bool NT>
__device__ __forceinline__ uint4 ld_row16(const uint16_t* row, uint32_t lane_bytes) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t* p = reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(row) + lane_bytes);
  const u32x4_t v = NT ? __builtin_nontemporal_load(p) : *p;
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Loads of the U tokens j..j+U-1 of this wave.  Loads are unconditional
// (tokens past the wave's end repeat its last token, absent ones read the
// cache's first row) so that all are in flight at once; consume skips both
// entirely, so no value of those rows (NaN included) reaches the result.
template <int U, bool NT>
__device__ __forceinline__ void issue_loads(const AttnArgs& a, const WaveRows& wr, int j, uint32_t lane_bytes,
                                            int64_t (&off)[U], uint4 (&kr)[U], uint4 (&vr)[U]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    off[u] = row_off(wr, j + u);
    const int64_t o = max(off[u], (int64_t)0);
    kr[u] = ld_row16<NT>(a.kc + o, lane_bytes);
    vr[u] = ld_row16<NT>(a.vc + o, lane_bytes);
  }
}

// Online-softmax update with one stage of U tokens: the U dot products and
// their DPP reductions are independent (they overlap), then the running max,
// sum and accumulator are rescaled once for the whole stage.
// q . k over a lane's 8 dims straight from the packed bf16 pairs
// (v_dot2_f32_bf16: both products exact in fp32), two chains for ILP
__device__ __forceinline__ float dot8_bf16(const uint4& q, const uint4& k) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  auto p = [](uint32_t x) { return __builtin_bit_cast(bf16x2_t, x); };
  float d0 = __builtin_amdgcn_fdot2_f32_bf16(p(q.x), p(k.x), 0.f, false);
  float d1 = __builtin_amdgcn_fdot2_f32_bf16(p(q.y), p(k.y), 0.f, false);
  d0 = __builtin_amdgcn_fdot2_f32_bf16(p(q.z), p(k.z), d0, false);
  d1 = __builtin_amdgcn_fdot2_f32_bf16(p(q.w), p(k.w), d1, false);
  return d0 + d1;
}

template <int D, int GQ, int U>
__device__ __forceinline__ void consume(const WaveRows& wr, int j, const int64_t (&off)[U], float scale_log2,
                                        const uint4 (&qv)[GQ], float (&m)[GQ], float (&l)[GQ],
                                        float (&acc)[GQ][8], const uint4 (&kr)[U], const uint4 (&vr)[U]) {
  constexpr int SLOT = D / 8;
  bool ok[U];
#pragma unroll
  for (int u = 0; u < U; ++u) ok[u] = j + u < wr.nw && off[u] >= 0;   // wave-uniform
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      sc[u] = group_sum_dpp<SLOT>(dot8_bf16(qv[j], kr[u])) * scale_log2;
    }
    float smax = m[j];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (ok[u]) smax = fmaxf(smax, sc[u]);
    if (smax == -INFINITY) continue;   // nothing valid yet (wave-uniform)
    const float corr = fast_exp2(m[j] - smax);
    float lsum = l[j] * corr;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = acc[j][e] * corr;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!ok[u]) continue;
      const float p = fast_exp2(sc[u] - smax);
      lsum += p;
      o[0] = fmaf(p, bf16_lo(vr[u].x), o[0]);
      o[1] = fmaf(p, bf16_hi(vr[u].x), o[1]);
      o[2] = fmaf(p, bf16_lo(vr[u].y), o[2]);
      o[3] = fmaf(p, bf16_hi(vr[u].y), o[3]);
      o[4] = fmaf(p, bf16_lo(vr[u].z), o[4]);
      o[5] = fmaf(p, bf16_hi(vr[u].z), o[5]);
      o[6] = fmaf(p, bf16_lo(vr[u].w), o[6]);
      o[7] = fmaf(p, bf16_hi(vr[u].w), o[7]);
    }
    l[j] = lsum;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = o[e];
    m[j] = smax;
  }
}

template <int D, int GQ, int U, bool NT, int W = kWaves>
__global__ __launch_bounds__(W * 64) void mha_attn_kernel(AttnArgs a) {
  constexpr int SLOT = D / 8;            // lanes per KV row
  constexpr int NSLOT = 64 / SLOT;       // KV heads per wave
  constexpr int NH = NSLOT * GQ;         // query heads per workgroup
  constexpr int NTH = W * 64;
  __shared__ float s_ml[W][NH][2];
  __shared__ float s_o[W][NH][D];

  int split, hg, bs;
  if (a.row_grouped) {
    // Several query rows (the verify pass): workgroups are dealt to the 8
    // XCDs round-robin by linear id, so XCD x's k-th workgroup takes row
    // k % S_q of unit (k / S_q) * 8 + x.  The S_q rows of a unit (same
    // sequence, split and head group) then run on one XCD at about the same
    // time, and rows with (nearly) the same index set read the same KV rows
    // through that XCD's L2.
    const int id = blockIdx.x;
    const int slot = id >> 3;
    const int unit = (slot / a.S_q) * 8 + (id & 7);
    const int s_row = slot % a.S_q;
    const int per_seq = a.nsplit * a.head_groups;
    if (unit >= a.batch * per_seq) return;          // padding of the unit count to a multiple of 8
    const int bb = unit / per_seq;
    split = (unit % per_seq) / a.head_groups;
    hg = unit % a.head_groups;
    bs = bb * a.S_q + s_row;
  } else {
    split = blockIdx.x;
    hg = blockIdx.y;                                 // KV head group
    bs = blockIdx.z;                                 // b * S_q + s
  }
  const int b = bs / a.S_q;
  const int s = bs % a.S_q;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int slot = lane / SLOT;
  const int sub = lane % SLOT;
  const int g = hg * NSLOT + slot;                   // KV head of this lane
  const bool head_ok = g < a.H_kv;

  // Row offsets of this wave's tokens (split-local w, w + W, ...),
  // resolved through the page table once, two per lane; no barrier.
  const int32_t* idx = a.idx + ((size_t)b * a.idx_rows + (a.idx_rows > 1 ? s : 0)) * a.k;
  const int32_t* bt = a.bt + (size_t)b * a.max_pages;
  const int t_lo = split * a.tok_per_split;
  const int ntok = min(a.tok_per_split, a.k - t_lo);
  WaveRows wr;
  wr.nw = wave < ntok ? (ntok - wave + W - 1) / W : 0;
  // Both of the lane's tokens at once: the two index loads (clamped inside
  // the index row) and the query loads, then the two block-table loads
  // (entry 0 for an absent token), so the start-up is two round trips, not
  // two per token.  Absent tokens, and positions outside the block table
  // (outside the contract), resolve to -1.
  const int ja = t_lo + wave + lane * W;
  const int jb = ja + 64 * W;
  const int ta = idx[min(ja, a.k - 1)];
  const int tb = idx[min(jb, a.k - 1)];
  uint4 qv[GQ];   // this lane's 8 query dims per head, packed bf16 pairs (0 for a padding head)
  const uint32_t qkeep = head_ok ? ~0u : 0u;
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    const uint4 v =
        *reinterpret_cast<const uint4*>(a.q + ((size_t)bs * a.H_q + min(g, a.H_kv - 1) * GQ + j) * D + sub * 8);
    qv[j] = make_uint4(v.x & qkeep, v.y & qkeep, v.z & qkeep, v.w & qkeep);
  }
  // page and in-page row of each token, computed unconditionally (unsigned)
  const uint32_t ua = (uint32_t)max(ta, 0), ub = (uint32_t)max(tb, 0);
  const uint32_t pga = ua / (uint32_t)a.page, pgb = ub / (uint32_t)a.page;
  const uint32_t ina = ua - pga * (uint32_t)a.page, inb = ub - pgb * (uint32_t)a.page;
  const bool oka = lane < wr.nw && ta >= 0 && pga < (uint32_t)a.max_pages;
  const bool okb = lane + 64 < wr.nw && tb >= 0 && pgb < (uint32_t)a.max_pages;
  const int pa = bt[oka ? pga : 0u];
  const int pb = bt[okb ? pgb : 0u];
  const int64_t offa = (int64_t)pa * a.page_stride + (int64_t)ina * a.row_stride;
  const int64_t offb = (int64_t)pb * a.page_stride + (int64_t)inb * a.row_stride;
  wr.o0 = oka ? offa : (int64_t)-1;
  wr.o1 = okb ? offb : (int64_t)-1;
  float m[GQ], l[GQ], acc[GQ][8];
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  }
  // Wave w takes split-local tokens w, w + W, ... (its local tokens
  // 0, 1, ...); loads run one U-token stage ahead.  Padding heads
  // (g >= H_kv) read the last real head; their results are dropped.
  const uint32_t lane_bytes = (uint32_t)(((int64_t)min(g, a.H_kv - 1) * a.head_stride + sub * 8) * 2);
  uint4 kA[U], vA[U], kB[U], vB[U];
  int64_t oA[U], oB[U];
  int j = 0;
  issue_loads<U, NT>(a, wr, j, lane_bytes, oA, kA, vA);
  while (j < wr.nw) {
    issue_loads<U, NT>(a, wr, j + U, lane_bytes, oB, kB, vB);
    consume<D, GQ, U>(wr, j, oA, a.scale_log2, qv, m, l, acc, kA, vA);
    j += U;
    if (j >= wr.nw) break;
    issue_loads<U, NT>(a, wr, j + U, lane_bytes, oA, kA, vA);
    consume<D, GQ, U>(wr, j, oB, a.scale_log2, qv, m, l, acc, kB, vB);
    j += U;
  }

  // merge the waves (fixed order)
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    if (sub == 0) {
      s_ml[wave][slot * GQ + j][0] = m[j];
      s_ml[wave][slot * GQ + j][1] = l[j];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s_o[wave][slot * GQ + j][sub * 8 + e] = acc[j][e];
  }
  __syncthreads();
  for (int p = tid; p < NH * D; p += NTH) {
    const int hj = p / D;
    const int d = p % D;
    const int gg = hg * NSLOT + hj / GQ;
    if (gg >= a.H_kv) continue;
    const int h = gg * GQ + hj % GQ;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, s_ml[w][hj][0]);
    float Lsum = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float c = fast_exp2(s_ml[w][hj][0] - M);
        Lsum += c * s_ml[w][hj][1];
        O += c * s_o[w][hj][d];
      }
    }
    const size_t row = (size_t)bs * a.H_q + h;
    if (a.nsplit == 1) {
      a.out[row * D + d] = M == -INFINITY ? 0.f : O / Lsum;
      if (d == 0 && a.lse) a.lse[row] = M == -INFINITY ? -INFINITY : (M + __log2f(Lsum)) * kLn2;
    } else {
      a.part_o[(row * a.nsplit + split) * D + d] = O;
      if (d == 0) {
        a.part_ml[(row * a.nsplit + split) * 2 + 0] = M;
        a.part_ml[(row * a.nsplit + split) * 2 + 1] = Lsum;
      }
    }
  }
}

// Folds split partials in split order: one workgroup per (b, s, h) row and
// DW output dims.  The split statistics (m, l) are the
// same for every thread of the row (scalar loads); each thread issues the
// loads of all its split partials at once, so the fold is one memory round
// trip with no barrier.
constexpr int kCombineMaxSplits = 128;
#ifndef DSA_LAT_MAX_SPLITS
#define DSA_LAT_MAX_SPLITS 32
#endif
#ifndef DSA_LAT_MIN_TOKENS
#define DSA_LAT_MIN_TOKENS 64
#endif
constexpr int kLatentMaxSplits = DSA_LAT_MAX_SPLITS;

template <int N>
struct FVec;
template <>
struct FVec<1> {
  typedef float T;
  static __device__ __forceinline__ T zero() { return 0.f; }
};
template <>
struct FVec<4> {
  typedef float4 T;
  static __device__ __forceinline__ T zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
};
__device__ __forceinline__ void fma_into(float& o, float c, float v) { o += c * v; }
__device__ __forceinline__ void fma_into(float4& o, float c, const float4& v) {
  o.x += c * v.x;
  o.y += c * v.y;
  o.z += c * v.z;
  o.w += c * v.w;
}
__device__ __forceinline__ float div_by(float o, float l) { return o / l; }
__device__ __forceinline__ float4 div_by(const float4& o, float l) {
  return make_float4(o.x / l, o.y / l, o.z / l, o.w / l);
}

// DW output dims per workgroup, VEC of them per thread
template <int D, int DW, int VEC, int MAXSPLIT>
__global__ __launch_bounds__(DW / VEC) void combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml, int nsplit,
                                                           float* __restrict__ out, float* __restrict__ lse) {
  typedef typename FVec<VEC>::T vec_t;
  const int row = blockIdx.x;
  const int d = blockIdx.y * DW + threadIdx.x * VEC;
  const float* ml = part_ml + (size_t)row * nsplit * 2;
  const float* po = part_o + (size_t)row * nsplit * D + d;
  vec_t ov[MAXSPLIT];
  float mv[MAXSPLIT], lv[MAXSPLIT];
#pragma unroll
  for (int sp = 0; sp < MAXSPLIT; ++sp) {
    const int c = min(sp, nsplit - 1);
    ov[sp] = *reinterpret_cast<const vec_t*>(po + (size_t)c * D);
    mv[sp] = ml[2 * c];
    lv[sp] = ml[2 * c + 1];
  }
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < MAXSPLIT; ++sp)
    if (sp < nsplit) M = fmaxf(M, mv[sp]);
  vec_t O = FVec<VEC>::zero();
  float Lsum = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int sp = 0; sp < MAXSPLIT; ++sp) {
      if (sp < nsplit) {
        const float c = fast_exp2(mv[sp] - M);
        fma_into(O, c, ov[sp]);
        Lsum += c * lv[sp];
      }
    }
  }
  *reinterpret_cast<vec_t*>(out + (size_t)row * D + d) = M == -INFINITY ? FVec<VEC>::zero() : div_by(O, Lsum);
  if (d == 0 && lse) lse[row] = M == -INFINITY ? -INFINITY : (M + __log2f(Lsum)) * kLn2;
}

// D output dims per row, DW of them per workgroup (rows x D/DW workgroups),
// VEC per thread: 16-byte accesses for the 64/128-dim rows; the 512-dim
// latent rows keep one dim per thread, spread over four workgroups per row
template <int D, int DW = (D < 128 ? D : 128), int VEC = (D <= 128 ? 4 : 1)>
void launch_combine(const float* part_o, const float* part_ml, int rows, int nsplit, float* out, float* lse,
                    hipStream_t s) {
  const dim3 grid(rows, D / DW), block(DW / VEC);
  if (nsplit <= 8)
    hipLaunchKernelGGL((combine_kernel<D, DW, VEC, 8>), grid, block, 0, s, part_o, part_ml, nsplit, out, lse);
  else if (nsplit <= 16)
    hipLaunchKernelGGL((combine_kernel<D, DW, VEC, 16>), grid, block, 0, s, part_o, part_ml, nsplit, out, lse);
  else if (nsplit <= 32)
    hipLaunchKernelGGL((combine_kernel<D, DW, VEC, 32>), grid, block, 0, s, part_o, part_ml, nsplit, out, lse);
  else if (nsplit <= 64)
    hipLaunchKernelGGL((combine_kernel<D, DW, VEC, 64>), grid, block, 0, s, part_o, part_ml, nsplit, out, lse);
  else
    hipLaunchKernelGGL((combine_kernel<D, DW, VEC, 128>), grid, block, 0, s, part_o, part_ml, nsplit, out, lse);
}

// ---------------------------------------------------------------------------
// Latent MQA kernel: one KV head of D_qk = 576 (K = the whole row, V = its
// first 512 dims) shared by 64 query heads.  A workgroup owns one split of the
// selected tokens and one group of 16 heads (the grid also runs over the four
// head groups, so a split's partial is 16 x 512 floats, and 128 workgroups run
// at k = 2048).  Per 64-token chunk, four waves:
//   * wave w loads the K rows of tokens 16w..16w+15 straight into B fragments
//     and computes S = Q K^T for them (18 K-steps of v_mfma_f32_16x16x32_bf16);
//   * every thread loads V pieces (lane = token) and writes them transposed
//     into LDS, so the PV operand is one 16-byte LDS read;
//   * the chunk's softmax statistics are combined across the waves in LDS
//     (online over chunks, exp2 domain), P goes to LDS as bf16;
//   * wave w accumulates O[16 heads][dims 128w..128w+127] += P V.
// Split-k partials (unnormalised O, m, l) go to the combine kernel as in the
// per-head kernel.
// ---------------------------------------------------------------------------
constexpr int kLatD = 576;
constexpr int kLatDv = 512;
constexpr int kLatChunk = 64;                     // tokens per chunk (4 waves x 16)
constexpr int kLatHeads = 16;                     // heads per workgroup
constexpr int kLatVRow = kLatChunk * 2 + 16;      // bytes per transposed V row in LDS (padded)
constexpr int kLatPRow = kLatChunk + 8;           // bf16 per P row in LDS (padded)

template <int CTRL>
__device__ __forceinline__ float dpp_max_step(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xf, 0xf, false)));
}
__device__ __forceinline__ float group_max16(float v) {
  v = dpp_max_step<0xB1>(v);
  v = dpp_max_step<0x4E>(v);
  v = dpp_max_step<0x141>(v);
  v = dpp_max_step<0x140>(v);
  return v;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rn(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);   // round to nearest even (finite inputs)
  return (uint16_t)(u >> 16);
}

__global__ __launch_bounds__(256) void latent_attn_kernel(AttnArgs a) {
  constexpr int NT = 256;
  constexpr int KS = kLatD / 32;                   // 18 K-steps of QK
  constexpr int DV_W = kLatDv / 4;                 // value dims per wave
  constexpr int NBV = DV_W / 16;                   // N-blocks of PV per wave
  constexpr int VPT = kLatChunk * (kLatDv / 8) / NT;   // 16-byte V pieces per thread per chunk (16)
  __shared__ int64_t s_off[kMaxTokPerSplit];
  __shared__ __align__(16) unsigned char s_vt[kLatDv * kLatVRow];
  __shared__ __align__(16) uint16_t s_p[kLatHeads][kLatPRow];
  __shared__ float s_wmax[4][kLatHeads], s_wsum[4][kLatHeads];

  const int split = blockIdx.x;
  const int hg = blockIdx.y;
  const int bs = blockIdx.z;
  const int b = bs / a.S_q;
  const int s = bs % a.S_q;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r16 = lane & 15;
  const int grp = lane >> 4;

  const int32_t* idx = a.idx + ((size_t)b * a.idx_rows + (a.idx_rows > 1 ? s : 0)) * a.k;
  const int32_t* bt = a.bt + (size_t)b * a.max_pages;
  const int t_lo = split * a.tok_per_split;
  const int ntok = min(a.tok_per_split, a.k - t_lo);
  for (int i = tid; i < ntok; i += NT) {
    const int t = idx[t_lo + i];
    // positions outside the block table (outside the contract) count as absent
    s_off[i] = (t >= 0 && t / a.page < a.max_pages) ? (int64_t)bt[t / a.page] * a.page_stride + (int64_t)(t % a.page) * a.row_stride : -1;
  }
  // Q fragments (A operand): lane holds head 16hg + l%16, dims ks*32 + (l/16)*8 .. +8
  bf16x8_t qa[KS];
  {
    const uint16_t* qrow = a.q + ((size_t)bs * a.H_q + hg * kLatHeads + r16) * kLatD + grp * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 32);
  }
  // accumulators: lane holds heads 4*grp + i, dims 128w + nb*16 + l%16
  f32x4_t o[NBV];
#pragma unroll
  for (int nb = 0; nb < NBV; ++nb) o[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
  }
  __syncthreads();

  const int nchunks = (ntok + kLatChunk - 1) / kLatChunk;
  for (int ch = 0; ch < nchunks; ++ch) {
    const int c0 = ch * kLatChunk;
    // V pieces: lane = token c0 + lane, dim chunk wave + 4j.  Loads are
    // unconditional (absent tokens and tokens past ntok read the cache's first
    // row), then such tokens' pieces are replaced by zeros: their softmax
    // weight is exactly 0, but 0 * NaN (a draft-written, unused or
    // uninitialised row) would still reach every head's output through PV.
    uint4 vp[VPT];
    {
      const int li = min(c0 + lane, ntok - 1);
      const int64_t off = max(s_off[li], (int64_t)0);
      const bool vok = c0 + lane < ntok && s_off[li] >= 0;
#pragma unroll
      for (int j = 0; j < VPT; ++j) vp[j] = *reinterpret_cast<const uint4*>(a.kc + off + (wave + 4 * j) * 8);
#pragma unroll
      for (int j = 0; j < VPT; ++j)
        if (!vok) vp[j] = make_uint4(0u, 0u, 0u, 0u);
    }
    // K fragments of this wave's 16 tokens (B operand): lane holds token
    // c0 + 16w + l%16, dims ks*32 + (l/16)*8 .. +8.  An absent token's K row
    // only feeds its own column of S, which is replaced by -inf below.
    const int my_tok = c0 + wave * 16 + r16;
    const bool valid = my_tok < ntok && s_off[min(my_tok, ntok - 1)] >= 0;
    bf16x8_t kf[KS];
    {
      const int64_t off = max(s_off[min(my_tok, ntok - 1)], (int64_t)0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[ks] = *reinterpret_cast<const bf16x8_t*>(a.kc + off + ks * 32 + grp * 8);
    }
    // V transposed into LDS: one instruction writes 64 consecutive tokens of one dim
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int d0 = (wave + 4 * j) * 8;
      const uint32_t w4[4] = {vp[j].x, vp[j].y, vp[j].z, vp[j].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t v = (uint16_t)(e & 1 ? (w4[e >> 1] >> 16) : (w4[e >> 1] & 0xffffu));
        *reinterpret_cast<uint16_t*>(s_vt + (d0 + e) * kLatVRow + lane * 2) = v;
      }
    }
    // S for heads 4*grp + i, token 16w + l%16
    f32x4_t sacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kf[ks], sacc, 0, 0, 0);
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = valid ? sacc[i] * a.scale_log2 : -INFINITY;
      const float wm = group_max16(sv[i]);
      if (r16 == 0) s_wmax[wave][grp * 4 + i] = wm;
    }
    __syncthreads();
    // chunk statistics, the same in every wave (fixed wave order)
    float corr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = grp * 4 + i;
      const float cm = fmaxf(fmaxf(s_wmax[0][h], s_wmax[1][h]), fmaxf(s_wmax[2][h], s_wmax[3][h]));
      const float mn = fmaxf(m_run[i], cm);
      corr[i] = mn == -INFINITY ? 1.f : fast_exp2(m_run[i] - mn);
      const uint16_t pb = f32_to_bf16_rn(mn == -INFINITY ? 0.f : fast_exp2(sv[i] - mn));
      // the row sum uses the bf16-rounded weights that PV multiplies
      const float ws = group_sum_dpp<16>(__uint_as_float((uint32_t)pb << 16));
      if (r16 == 0) s_wsum[wave][h] = ws;
      s_p[h][wave * 16 + r16] = pb;
      m_run[i] = mn;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = grp * 4 + i;
      l_run[i] = l_run[i] * corr[i] + ((s_wsum[0][h] + s_wsum[1][h]) + (s_wsum[2][h] + s_wsum[3][h]));
    }
    // O[16 heads][this wave's dims] = O * corr + P V  (two 32-token K-steps)
    bf16x8_t pa[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) pa[kk] = *reinterpret_cast<const bf16x8_t*>(&s_p[r16][kk * 32 + grp * 8]);
#pragma unroll
    for (int nb = 0; nb < NBV; ++nb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[nb][i] *= corr[i];
      const unsigned char* vrow = s_vt + (wave * DV_W + nb * 16 + r16) * kLatVRow + grp * 16;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[kk], *reinterpret_cast<const bf16x8_t*>(vrow + kk * 64),
                                                       o[nb], 0, 0, 0);
    }
    __syncthreads();   // the next chunk overwrites s_vt, s_p and the statistics
  }

  // every wave holds the same statistics; wave 0 writes them
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const size_t row = (size_t)bs * a.H_q + hg * kLatHeads + grp * 4 + i;
    if (wave == 0 && r16 == 0) {
      if (a.nsplit == 1) {
        if (a.lse) a.lse[row] = m_run[i] == -INFINITY ? -INFINITY : (m_run[i] + __log2f(l_run[i])) * kLn2;
      } else {
        a.part_ml[(row * a.nsplit + split) * 2 + 0] = m_run[i];
        a.part_ml[(row * a.nsplit + split) * 2 + 1] = l_run[i];
      }
    }
    const float inv = l_run[i] > 0.f ? 1.f / l_run[i] : 0.f;
#pragma unroll
    for (int nb = 0; nb < NBV; ++nb) {
      const int dv = wave * DV_W + nb * 16 + r16;
      if (a.nsplit == 1) a.out[row * kLatDv + dv] = o[nb][i] * inv;
      else a.part_o[(row * a.nsplit + split) * kLatDv + dv] = o[nb][i];
    }
  }
}

// ---------------------------------------------------------------------------
// Launch planning (shared by the workspace query and the call)
// ---------------------------------------------------------------------------
struct Plan {
  int nsplit;
  int tok_per_split;
  int head_groups;
  size_t ws_bytes;
  size_t part_o_off, part_ml_off;
};

// The latent kernel is instantiated for 64 query heads (4 waves); fewer
// heads would leave its per-wave register tiles spilling.
bool is_latent(int H_q, int H_kv, int D_qk, int D_v) {
  return H_kv == 1 && D_qk == kLatD && D_v == kLatDv && H_q == 64;
}

// One query row per sequence and a per-head-KV gather larger than the
// last-level cache: the KV rows are streamed with non-temporal loads (no
// draft step re-reads them from that cache).
bool streams_kv(int B, int S_q, int H_kv, int D, int k) {
  return S_q == 1 && (double)B * k * H_kv * D * 2 * 2 > (double)kAttnStreamBytes;
}

// The streamed gather runs kStreamWaves per workgroup when each KV head has
// one query head (the per-wave merge buffers then fit in LDS).
bool wide_stream(int B, int S_q, int H_q, int H_kv, int D, int k) {
  return H_q == H_kv && streams_kv(B, S_q, H_kv, D, k);
}

Plan make_plan(int B, int S_q, int H_q, int H_kv, int D_qk, int D_v, int k) {
  Plan p{};
  const bool latent = is_latent(H_q, H_kv, D_qk, D_v);
  const int nslot = latent ? 1 : 64 / (D_qk / 8);
  p.head_groups = latent ? H_q / kLatHeads : (H_kv + nslot - 1) / nslot;
  const long long base = (long long)B * S_q * p.head_groups;
  const int min_tok = latent ? DSA_LAT_MIN_TOKENS : DSA_ATTN_MIN_TOKENS;
  const int max_split = latent ? kLatentMaxSplits : kCombineMaxSplits;
  // a streamed gather keeps every CU busy with one workgroup per (sequence,
  // head group) once there are about 256 of them: no split, no combine
  const long long target = (!latent && streams_kv(B, S_q, H_kv, D_qk, k)) ? DSA_ATTN_TARGET_WGS_STREAM
                                                                         : DSA_ATTN_TARGET_WGS;
  int ns = (int)((target + base - 1) / base);
  const int max_ns = (k + min_tok - 1) / min_tok;
  if (ns > max_ns) ns = max_ns;
  const int max_tok = (!latent && wide_stream(B, S_q, H_q, H_kv, D_qk, k)) ? kStreamTokPerSplit : kMaxTokPerSplit;
  const int min_ns = (k + max_tok - 1) / max_tok;
  if (ns < min_ns) ns = min_ns;
  if (ns > max_split) ns = max_split;
  if (ns < 1) ns = 1;
  p.tok_per_split = (k + ns - 1) / ns;
  p.nsplit = (k + p.tok_per_split - 1) / p.tok_per_split;
  const size_t rows = (size_t)B * S_q * H_q;
  if (p.nsplit > 1) {
    p.part_o_off = 0;
    p.part_ml_off = p.part_o_off + align_up(rows * p.nsplit * D_v * sizeof(float), 256);
    p.ws_bytes = p.part_ml_off + align_up(rows * p.nsplit * 2 * sizeof(float), 256);
  }
  return p;
}

template <int D, int GQ>
void launch_mha(AttnArgs a, const Plan& p, int B, hipStream_t s) {
  a.batch = B;
  a.head_groups = p.head_groups;
  if (a.S_q > 1) {
    // flat grid: units (b, split, head group) padded to a multiple of the 8
    // XCDs, times S_q rows (see the kernel)
    const long long units = ((long long)B * p.nsplit * p.head_groups + 7) / 8 * 8;
    a.row_grouped = 1;
    hipLaunchKernelGGL((mha_attn_kernel<D, GQ, DSA_ATTN_UNROLL, false>), dim3((unsigned)(units * a.S_q)),
                       dim3(kThreads), 0, s, a);
  } else {
    a.row_grouped = 0;
    dim3 grid(p.nsplit, p.head_groups, B * a.S_q);
    // one query row per sequence: a gather larger than the last-level cache
    // streams (non-temporal loads, four tokens per stage, about 256
    // workgroups); smaller ones stay cacheable, since the draft steps that
    // share the index set re-read the same rows
    if (streams_kv(B, a.S_q, a.H_kv, D, a.k)) {
      if constexpr (GQ == 1) {
        // 16 waves: one workgroup per (sequence, head group) for k <= 2048
        if (wide_stream(B, a.S_q, a.H_q, a.H_kv, D, a.k)) {
          hipLaunchKernelGGL((mha_attn_kernel<D, GQ, DSA_ATTN_UNROLL_NT, true, kStreamWaves>), grid,
                             dim3(kStreamWaves * 64), 0, s, a);
          return;
        }
      }
      hipLaunchKernelGGL((mha_attn_kernel<D, GQ, DSA_ATTN_UNROLL_NT, true>), grid, dim3(kThreads), 0, s, a);
    } else {
      hipLaunchKernelGGL((mha_attn_kernel<D, GQ, DSA_ATTN_UNROLL, false>), grid, dim3(kThreads), 0, s, a);
    }
  }
}

}  // namespace
}  // namespace dsa

extern "C" size_t dsa_sparse_attn_workspace_size(int B, int S_q, int H_q, int H_kv, int D_qk, int D_v, int k) {
  if (B < 1 || S_q < 1 || H_q < 1 || H_kv < 1 || D_qk < 8 || D_v < 1 || k < 1) return 0;
  if (D_qk != 64 && D_qk != 128 && !dsa::is_latent(H_q, H_kv, D_qk, D_v)) return 0;
  return dsa::make_plan(B, S_q, H_q, H_kv, D_qk, D_v, k).ws_bytes;
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point: the split-k partials live in a
// file-scope device array instead of a caller workspace.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: its device address
// is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is ever passed to kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];

namespace dsa {
namespace {

// Host-side argument checks shared by both entry points (no HIP call).
dsa_status check_args(const char* fn, const void* q, const void* k_cache, const void* v_cache,
                      int64_t kv_page_stride, int64_t kv_row_stride, int64_t kv_head_stride,
                      const int32_t* block_table, const int32_t* idx, int idx_rows, int B, int S_q, int H_q,
                      int H_kv, int D_qk, int D_v, int page, int max_pages, int k, float sm_scale,
                      const float* out) {
  DSA_REQUIRE(q && k_cache && v_cache && block_table && idx && out, DSA_ERR_INVALID_ARG,
              "%s: null pointer argument", fn);
  DSA_REQUIRE(B >= 1 && S_q >= 1 && H_q >= 1 && H_kv >= 1 && D_qk >= 1 && D_v >= 1 && page >= 1 &&
                  max_pages >= 1 && k >= 1,
              DSA_ERR_INVALID_ARG, "%s: sizes must be positive", fn);
  DSA_REQUIRE((int64_t)B * S_q <= 65535, DSA_ERR_UNSUPPORTED, "%s: B*S_q=%lld > 65535", fn,
              (long long)B * S_q);
  DSA_REQUIRE(idx_rows == 1 || idx_rows == S_q, DSA_ERR_INVALID_ARG,
              "%s: idx_rows=%d must be 1 or S_q=%d", fn, idx_rows, S_q);
  DSA_REQUIRE(kv_page_stride >= 0 && kv_row_stride >= 0 && kv_head_stride >= 0, DSA_ERR_INVALID_ARG,
              "%s: strides must be non-negative", fn);
  DSA_REQUIRE(H_q % H_kv == 0, DSA_ERR_INVALID_ARG, "%s: H_q=%d not a multiple of H_kv=%d", fn, H_q, H_kv);
  DSA_REQUIRE(std::isfinite(sm_scale), DSA_ERR_INVALID_ARG, "%s: sm_scale not finite", fn);
  const int gq = H_q / H_kv;
  const bool latent = is_latent(H_q, H_kv, D_qk, D_v);
  DSA_REQUIRE(latent || ((D_qk == 64 || D_qk == 128) && D_v == D_qk && (gq == 1 || gq == 2 || gq == 4)),
              DSA_ERR_UNSUPPORTED, "%s: (H_q=%d, H_kv=%d, D_qk=%d, D_v=%d) not supported", fn,
              H_q, H_kv, D_qk, D_v);
  DSA_REQUIRE(!latent || v_cache == k_cache, DSA_ERR_UNSUPPORTED,
              "%s: the latent path reads V from the key rows (pass v_cache == k_cache)", fn);
  DSA_REQUIRE(k <= (latent ? kLatentMaxSplits : kCombineMaxSplits) * kMaxTokPerSplit, DSA_ERR_UNSUPPORTED,
              "%s: k=%d too large", fn, k);
  DSA_REQUIRE(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned16(out) &&
                  kv_page_stride % 8 == 0 && kv_row_stride % 8 == 0 && kv_head_stride % 8 == 0,
              DSA_ERR_INVALID_ARG, "%s: q/K/V rows and out must be 16-byte aligned", fn);
  return DSA_OK;
}

// Enqueues the call once the arguments are checked; `ws` holds at least
// p.ws_bytes bytes of device memory when p.ws_bytes > 0.
dsa_status enqueue(const Plan& p, const void* q, const void* k_cache, const void* v_cache, int64_t kv_page_stride,
                   int64_t kv_row_stride, int64_t kv_head_stride, const int32_t* block_table, const int32_t* idx,
                   int idx_rows, int B, int S_q, int H_q, int H_kv, int D_qk, int D_v, int page, int max_pages,
                   int k, float sm_scale, float* out, float* lse, void* ws, hipStream_t s) {
  const int gq = H_q / H_kv;
  const bool latent = is_latent(H_q, H_kv, D_qk, D_v);
  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.kc = static_cast<const uint16_t*>(k_cache);
  a.vc = static_cast<const uint16_t*>(v_cache);
  a.page_stride = kv_page_stride;
  a.row_stride = kv_row_stride;
  a.head_stride = kv_head_stride;
  a.bt = block_table;
  a.idx = idx;
  a.idx_rows = idx_rows;
  a.S_q = S_q;
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.page = page;
  a.max_pages = max_pages;
  a.k = k;
  a.scale_log2 = sm_scale * kLog2e;
  a.out = out;
  a.lse = lse;
  a.nsplit = p.nsplit;
  a.tok_per_split = p.tok_per_split;
  if (p.nsplit > 1) {
    a.part_o = reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_o_off);
    a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_ml_off);
  }
  if (latent) {
    dim3 grid(p.nsplit, p.head_groups, B * S_q);
    hipLaunchKernelGGL(latent_attn_kernel, grid, dim3(256), 0, s, a);
    dsa_status st = launch_status("dsa_sparse_attn(latent)");
    if (st != DSA_OK || p.nsplit == 1) return st;
    launch_combine<kLatDv>(a.part_o, a.part_ml, B * S_q * H_q, p.nsplit, out, lse, s);
    return launch_status("dsa_sparse_attn(combine)");
  }
  if (D_qk == 64) {
    if (gq == 1) launch_mha<64, 1>(a, p, B, s);
    else if (gq == 2) launch_mha<64, 2>(a, p, B, s);
    else launch_mha<64, 4>(a, p, B, s);
  } else {
    if (gq == 1) launch_mha<128, 1>(a, p, B, s);
    else if (gq == 2) launch_mha<128, 2>(a, p, B, s);
    else launch_mha<128, 4>(a, p, B, s);
  }
  dsa_status st = launch_status("dsa_sparse_attn");
  if (st != DSA_OK || p.nsplit == 1) return st;
  const int rows = B * S_q * H_q;
  if (D_v == 64) launch_combine<64>(a.part_o, a.part_ml, rows, p.nsplit, out, lse, s);
  else launch_combine<128>(a.part_o, a.part_ml, rows, p.nsplit, out, lse, s);
  return launch_status("dsa_sparse_attn(combine)");
}

constexpr size_t kScratchBytes = DSA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

dsa_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  DSA_REQUIRE(e == hipSuccess, DSA_ERR_HIP, "dsa_sparse_attn_noalloc: hipGetDevice failed: %s",
              hipGetErrorString(e));
  DSA_REQUIRE(dev >= 0 && dev < kMaxDevices, DSA_ERR_UNSUPPORTED,
              "dsa_sparse_attn_noalloc: device %d beyond the %d devices supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    DSA_REQUIRE(e == hipSuccess && ptr, DSA_ERR_HIP,
                "dsa_sparse_attn_noalloc: hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace
}  // namespace dsa

extern "C" dsa_status dsa_sparse_attn(const void* q, const void* k_cache, const void* v_cache,
                                      int64_t kv_page_stride, int64_t kv_row_stride, int64_t kv_head_stride,
                                      const int32_t* block_table, const int32_t* idx, int idx_rows, int B,
                                      int S_q, int H_q, int H_kv, int D_qk, int D_v, int page, int max_pages,
                                      int k, float sm_scale, float* out, float* lse, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  using namespace dsa;
  clear_error();
  dsa_status st = check_args("dsa_sparse_attn", q, k_cache, v_cache, kv_page_stride, kv_row_stride, kv_head_stride,
                             block_table, idx, idx_rows, B, S_q, H_q, H_kv, D_qk, D_v, page, max_pages, k,
                             sm_scale, out);
  if (st != DSA_OK) return st;
  const Plan p = make_plan(B, S_q, H_q, H_kv, D_qk, D_v, k);
  DSA_REQUIRE(p.ws_bytes == 0 || (workspace && workspace_bytes >= p.ws_bytes), DSA_ERR_WORKSPACE,
              "dsa_sparse_attn: workspace of %zu bytes needed, %zu given", p.ws_bytes, workspace_bytes);
  return enqueue(p, q, k_cache, v_cache, kv_page_stride, kv_row_stride, kv_head_stride, block_table, idx, idx_rows,
                 B, S_q, H_q, H_kv, D_qk, D_v, page, max_pages, k, sm_scale, out, lse, workspace,
                 static_cast<hipStream_t>(stream));
}

extern "C" dsa_status dsa_sparse_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                              int64_t kv_page_stride, int64_t kv_row_stride,
                                              int64_t kv_head_stride, const int32_t* block_table,
                                              const int32_t* idx, int idx_rows, int B, int S_q, int H_q,
                                              int H_kv, int D_qk, int D_v, int page, int max_pages, int k,
                                              float sm_scale, float* out, float* lse, void* stream) {
  using namespace dsa;
  clear_error();
  dsa_status st = check_args("dsa_sparse_attn_noalloc", q, k_cache, v_cache, kv_page_stride, kv_row_stride,
                             kv_head_stride, block_table, idx, idx_rows, B, S_q, H_q, H_kv, D_qk, D_v, page,
                             max_pages, k, sm_scale, out);
  if (st != DSA_OK) return st;
  const Plan p = make_plan(B, S_q, H_q, H_kv, D_qk, D_v, k);
  DSA_REQUIRE(p.ws_bytes <= kScratchBytes, DSA_ERR_UNSUPPORTED,
              "dsa_sparse_attn_noalloc: this call needs %zu bytes of split-k scratch, more than the %zu bytes "
              "the allocation-free entry point holds (call dsa_sparse_attn with a workspace instead)",
              p.ws_bytes, kScratchBytes);
  void* ws = nullptr;
  if (p.ws_bytes > 0) {
    st = scratch_on_current_device(&ws);
    if (st != DSA_OK) return st;
  }
  return enqueue(p, q, k_cache, v_cache, kv_page_stride, kv_row_stride, kv_head_stride, block_table, idx, idx_rows,
                 B, S_q, H_q, H_kv, D_qk, D_v, page, max_pages, k, sm_scale, out, lse, ws,
                 static_cast<hipStream_t>(stream));
}
