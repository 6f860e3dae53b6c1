// Rejection-sampling verification of drafted chains (gfx950).
//
// Section "Rejection sampling and a loss that optimizes acceptance directly"
// ("Optimizing speculative decoding"): drafts sampled from the draft
// distribution q are accepted or rejected against the target distribution p,
// which preserves p.  Section "Kimi K3": sum_x min(p, q) is the exact
// per-token acceptance probability, i.e. d is accepted with probability
// min(1, p(d)/q(d)).  On the first rejection a token is drawn from
// norm(max(0, p - q)); if every draft is accepted a bonus token is drawn from
// the last target row.
//
// Four launches (three for at most 16 sequences, where the decision runs in
// every mass workgroup instead of a launch of its own):
//   stats   grid (chunk, row): the running max and sum of exp(x - max) of
//           each chunk of each of the 2G+1 rows of a sequence (fp32,
//           wavefront reductions), streamed once with 16-byte loads (whole
//           rows per workgroup when the batch fills the GPU; non-temporal
//           loads when the logits exceed the last-level cache).
//   decide  one workgroup per sequence folds its partials and tests the G
//           drafts in parallel lanes (first rejection by ballot).
//   mass    grid (chunk, sequence): the residual (or bonus) weights of one
//           chunk of the sampled row: per-256-logit tile masses from a wave
//           inclusive scan (kept in the workspace), added in tile order.
//   pick    one workgroup per sequence draws by inverse CDF: the chunk that
//           holds u * W, the tile inside it (from the stored tile masses),
//           then the token inside the tile.
// Batches of 1 GiB of logits or more take an early-exit schedule instead of
// the stats and decide launches: the protocol stops at the first rejection,
// so one launch per early position reads a position's two rows only for the
// chains still accepted (each workgroup first runs the accept test of the
// position before), and one last launch reads the remaining rows of the few
// chains that got that far; the mass kernel decides those, and pick is
// unchanged.  Greedy verification has the same two schedules.
// Uniforms come from the caller or from Philox4x64-10 (Salmon, Moraes, Dror,
// Shaw, SC'11) evaluated in-kernel at counter (offset, b, j, stream).
#include <cstdlib>
#include <cstring>

#include "dsa_common.h"

namespace dsa {
namespace {

#ifndef DSA_VERIFY_STAT_THREADS
#define DSA_VERIFY_STAT_THREADS 512
#endif
#ifndef DSA_VERIFY_STAT_U
#define DSA_VERIFY_STAT_U 2
#endif
constexpr int kStatThreads = DSA_VERIFY_STAT_THREADS;
constexpr int kStatU = DSA_VERIFY_STAT_U;       // float4 loads in flight per thread
constexpr int kStatStep = kStatThreads * 4;     // logits per load round of a workgroup
constexpr int kArgThreads = 256;                // greedy argmax pass: workgroup shape
constexpr int kArgU = 4;
constexpr int kArgStep = kArgThreads * 4;
#ifndef DSA_VERIFY_STAT_TARGET_WGS
#define DSA_VERIFY_STAT_TARGET_WGS 512
#endif
constexpr int kStatTargetWgs = DSA_VERIFY_STAT_TARGET_WGS;
// Early-exit (phased) verification: one launch per early position, each
// reading only the rows of the sequences whose chain is still accepted, then
// one for the rest.  It replaces the one-pass stats when the batch's logits
// reach this size (a few more dependent launches against the rows after each
// first rejection left unread).
#ifndef DSA_VERIFY_PHASED_MIN_MB
#define DSA_VERIFY_PHASED_MIN_MB 1024
#endif
constexpr size_t kPhasedMinBytes = (size_t)DSA_VERIFY_PHASED_MIN_MB << 20;
#ifndef DSA_VERIFY_PHASE_U
#define DSA_VERIFY_PHASE_U 4
#endif
constexpr int kPhaseU = DSA_VERIFY_PHASE_U;     // float4 loads in flight per thread in a phase
#ifndef DSA_VERIFY_PHASE_TARGET_WGS
#define DSA_VERIFY_PHASE_TARGET_WGS 2048
#endif
constexpr int kPhaseTargetWgs = DSA_VERIFY_PHASE_TARGET_WGS;   // workgroups of a phase when all sequences run
#ifndef DSA_VERIFY_PHASED_POSITIONS
#define DSA_VERIFY_PHASED_POSITIONS 4
#endif
constexpr int kPhasedPositions = DSA_VERIFY_PHASED_POSITIONS;   // positions with a launch of their own
#ifndef DSA_VERIFY_GREEDY_PHASED_POSITIONS
#define DSA_VERIFY_GREEDY_PHASED_POSITIONS 2
#endif
constexpr int kGreedyPhasedPositions = DSA_VERIFY_GREEDY_PHASED_POSITIONS;   // the same for greedy verification
constexpr int kPhaseFoldMax = 4;   // chunk partials per lane in a phase's accept test (up to 64 chunks a row)
constexpr size_t kStreamBytes = (size_t)256 << 20;   // above this, logits are streamed non-temporally
constexpr int kTile = 256;           // logits per wave step (64 lanes x 4)
constexpr int kMaxV = 1 << 20;
constexpr int kMaxTiles = kMaxV / kTile;
constexpr int kMaxG = 32;

__device__ __forceinline__ uint64_t philox4x64_10_first(uint64_t seed, uint64_t c0, uint64_t c1, uint64_t c2,
                                                        uint64_t c3) {
  uint64_t k0 = seed, k1 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B97F4A7C15ull;
      k1 += 0xBB67AE8584CAA73Bull;
    }
    const uint64_t lo0 = 0xD2E7470EE14C6C93ull * c0;
    const uint64_t hi0 = __umul64hi(0xD2E7470EE14C6C93ull, c0);
    const uint64_t lo1 = 0xCA5A826395121157ull * c2;
    const uint64_t hi1 = __umul64hi(0xCA5A826395121157ull, c2);
    const uint64_t n0 = hi1 ^ c1 ^ k0;
    const uint64_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return c0;
}

__device__ __forceinline__ float philox_uniform(uint64_t seed, uint64_t offset, int b, int j, int stream) {
  const uint64_t x = philox4x64_10_first(seed, offset, (uint64_t)b, (uint64_t)j, (uint64_t)stream);
  return (float)(x >> 40) * (1.0f / 16777216.0f);
}

// Merge of (max, sum exp(x - max)) pairs; empty = (-inf, 0).
__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  s = s * fast_exp2((m - M) * kLog2e) + s2 * fast_exp2((m2 - M) * kLog2e);
  m = M;
}

// 16-byte load; NT marks it non-temporal (streamed data that is not re-read soon)
template <bool NT>
__device__ __forceinline__ float4 ld16(const float* p) {
  const f32x4_t v = NT ? __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p))
                       : *reinterpret_cast<const f32x4_t*>(p);
  return make_float4(v[0], v[1], v[2], v[3]);
}

template <bool NT = false>
__device__ __forceinline__ float4 load4(const float* row, int e, int V, bool vec) {
  if (vec && e + 3 < V) return ld16<NT>(row + e);
  float4 r;
  r.x = e + 0 < V ? row[e + 0] : -INFINITY;
  r.y = e + 1 < V ? row[e + 1] : -INFINITY;
  r.z = e + 2 < V ? row[e + 2] : -INFINITY;
  r.w = e + 3 < V ? row[e + 3] : -INFINITY;
  return r;
}

struct VerifyArgs {
  const float* tl;
  const float* dl;
  const int32_t* drafts;
  int B, G, V, nchunks, chunk;
  const float* uniforms;
  uint64_t seed, offset;
  int32_t* acc_len;
  int32_t* emitted;
  float* diag;
  float2* part;        // [B][2G+1][nchunks]
  bool vec;
};

__device__ __forceinline__ const float* row_ptr(const VerifyArgs& a, int b, int r) {
  // rows 0..G: target rows; G+1..2G: draft rows 0..G-1
  if (r <= a.G) return a.tl + ((size_t)b * (a.G + 1) + r) * a.V;
  return a.dl + ((size_t)b * a.G + (r - a.G - 1)) * a.V;
}

template <bool NT>
__global__ __launch_bounds__(kStatThreads) void verify_stats_kernel(VerifyArgs a) {
  __shared__ float2 s_w[kStatThreads / 64];
  const int c = blockIdx.x;
  const int rr = blockIdx.y;                 // b * (2G+1) + r
  const int nrows = 2 * a.G + 1;
  const int b = rr / nrows;
  const int r = rr % nrows;
  const float* row = row_ptr(a, b, r);
  const int e0 = c * a.chunk;
  const int e1 = min(e0 + a.chunk, a.V);
  const float4 ninf = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
  float m = -INFINITY, s = 0.f;
  for (int e = e0 + threadIdx.x * 4; e < e1; e += kStatU * kStatStep) {
    float4 x[kStatU];
#pragma unroll
    for (int u = 0; u < kStatU; ++u) {
      const int ee = e + u * kStatStep;
      if (a.vec) {
        // unconditional aligned load (clamped inside the chunk), masked after
        const float4 v = ld16<NT>(row + (min(ee, e1 - 1) & ~3));
        x[u] = ee < e1 ? v : ninf;
      } else {
        x[u] = ee < e1 ? load4(row, ee, e1, false) : ninf;
      }
    }
    // one rescale per batch: max over the batch first, then its exponentials
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kStatU; ++u) bm = fmaxf(bm, fmaxf(fmaxf(x[u].x, x[u].y), fmaxf(x[u].z, x[u].w)));
    const float M = fmaxf(m, bm);
    if (M == -INFINITY) continue;   // nothing but -inf logits so far
    // exp(x - M) as 2^(x log2 e - M log2 e), one FMA per logit (the
    // exponent carries at most half an ulp of M log2 e: a relative error
    // below 3e-6 for |M| < 100)
    const float Mc = M * kLog2e;
    float t = 0.f;
#pragma unroll
    for (int u = 0; u < kStatU; ++u) {
      t += fast_exp2(fmaf(x[u].x, kLog2e, -Mc));
      t += fast_exp2(fmaf(x[u].y, kLog2e, -Mc));
      t += fast_exp2(fmaf(x[u].z, kLog2e, -Mc));
      t += fast_exp2(fmaf(x[u].w, kLog2e, -Mc));
    }
    s = s * fast_exp2((m - M) * kLog2e) + t;
    m = M;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64);
    const float s2 = __shfl_xor(s, o, 64);
    ms_merge(m, s, m2, s2);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) s_w[wave] = make_float2(m, s);
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = s_w[0].x, S = s_w[0].y;
    for (int w = 1; w < kStatThreads / 64; ++w) ms_merge(M, S, s_w[w].x, s_w[w].y);
    a.part[((size_t)b * nrows + r) * a.nchunks + c] = make_float2(M, S);
  }
}

// Weight of logit e of the sampled row (0 beyond V): p = softmax(t)_e and
// q = softmax(d)_e as 2^(x log2 e - o) with o = max * log2 e + log2(sum of
// exp(x - max)), one FMA and one exp2 each (the offsets are computed once per
// sequence).
struct RowWeights {
  const float* t;   // target row
  const float* d;   // draft row (residual) or nullptr (plain softmax of t)
  float ot, od;     // log2-domain offsets of the two rows
  __device__ __forceinline__ float w(float tv, float dv) const {
    const float p = fast_exp2(fmaf(tv, kLog2e, -ot));
    if (!d) return p;
    const float q = fast_exp2(fmaf(dv, kLog2e, -od));
    return fmaxf(p - q, 0.f);
  }
};

__device__ __forceinline__ float row_offset(float m, float z) { return m * kLog2e + log2f(z); }

__device__ __forceinline__ float wave_incl_scan(float v) { return wave_incl_scan_dpp(v); }

__device__ __forceinline__ void weights4(const RowWeights& rw, const float4& tv, const float4& dv, int e, int V,
                                         float wv[4]) {
  if (e + 3 < V) {   // whole quad inside the row: no per-logit checks
    wv[0] = rw.w(tv.x, dv.x);
    wv[1] = rw.w(tv.y, dv.y);
    wv[2] = rw.w(tv.z, dv.z);
    wv[3] = rw.w(tv.w, dv.w);
    return;
  }
  wv[0] = e + 0 < V ? rw.w(tv.x, dv.x) : 0.f;
  wv[1] = e + 1 < V ? rw.w(tv.y, dv.y) : 0.f;
  wv[2] = e + 2 < V ? rw.w(tv.z, dv.z) : 0.f;
  wv[3] = e + 3 < V ? rw.w(tv.w, dv.w) : 0.f;
}

// Per-lane weights of 4 consecutive logits and their wave inclusive scan.
__device__ __forceinline__ void tile_weights(const RowWeights& rw, int e, int V, bool vec, float wv[4],
                                             float& lane_incl) {
  const float4 tv = load4(rw.t, e, V, vec);
  float4 dv = make_float4(0.f, 0.f, 0.f, 0.f);
  if (rw.d) dv = load4(rw.d, e, V, vec);
  weights4(rw, tv, dv, e, V, wv);
  lane_incl = wave_incl_scan(((wv[0] + wv[1]) + wv[2]) + wv[3]);
}

// Per-sequence decision record written by the chunk-0 workgroup of the mass
// kernel: accepted length, sampling uniform and the sampled rows' softmax
// statistics.
struct Decision {
  int jstar;
  float us;
  float ot, od;     // RowWeights offsets of the sampled rows
  int pad0, pad1, pad2, pad3;
};

constexpr int kDecideThreads = 256;
#ifndef DSA_VERIFY_MASS_THREADS
#define DSA_VERIFY_MASS_THREADS 512
#endif
#ifndef DSA_VERIFY_BIG_CT
#define DSA_VERIFY_BIG_CT 32
#endif
constexpr int kMassThreads = DSA_VERIFY_MASS_THREADS;   // residual-mass workgroups
constexpr int kPickThreads = 1024;   // pick workgroups: 16 waves
constexpr int kSmallChunkTiles = 16;   // 4K-logit mass chunks (few sequences)
constexpr int kBigChunkTiles = DSA_VERIFY_BIG_CT;   // mass chunk tiles when there are many sequences
constexpr int kMaxMassChunks = kMaxV / (kSmallChunkTiles * kTile);

struct VerifyWs {
  float2* part;      // [B][2G+1][nchunks]
  Decision* dec;     // [B]
  float* cmass;      // [B][nmass]
  float* tmass;      // [B][ntiles]: tile masses of the sampled row
  int* reach;        // phased: [G+1][B], 1 where the chain reached position j
  float* dlog;       // phased: [B][G][2], target and draft logit of drafted token j
  int nmass;
  int ntiles;
  int chunk_tiles;   // 256-logit tiles per mass chunk
  bool phased;
  int tail;          // phased: first position of the last launch (one pass over its rows)
};

// Folds chunk partials (chunk order) and runs the accept tests for sequence
// b; results in shared memory.  Every workgroup of the sequence computes the
// same values from the same inputs.
__device__ void decide(const VerifyArgs& a, const VerifyWs& ws, int b, float* s_m, float* s_z, int* s_jstar,
                       float* s_us, bool write_diag) {
  const int G = a.G, V = a.V;
  const int nrows = 2 * G + 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the draft tokens' logits are fetched first so that their latency overlaps the fold
  float tv = 0.f, dv = 0.f;
  if (tid < G) {
    const int d = min(max(a.drafts[(size_t)b * G + lane], 0), V - 1);   // reads stay inside the row
    tv = a.tl[((size_t)b * (G + 1) + lane) * V + d];
    dv = a.dl[((size_t)b * G + lane) * V + d];
  }
  // 16 lanes per row, all rows at once (one round of loads): lane j of row
  // r's group merges chunks j, j + 16, ... in that order, then a 16-lane
  // butterfly (merging is symmetric, so every lane, and every workgroup of
  // the sequence, ends with the same bits)
  const int groups = blockDim.x / 16;
  const int g16 = tid >> 4, j16 = tid & 15;
  for (int r0 = 0; r0 < nrows; r0 += groups) {
    const int r = r0 + g16;
    float M = -INFINITY, S = 0.f;
    if (r < nrows) {
      const float2* p = ws.part + ((size_t)b * nrows + r) * a.nchunks;
      for (int c = j16; c < a.nchunks; c += 16) {
        const float2 v = p[c];
        ms_merge(M, S, v.x, v.y);
      }
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) {
      const float m2 = __shfl_xor(M, o, 64);
      const float s2 = __shfl_xor(S, o, 64);
      ms_merge(M, S, m2, s2);
    }
    if (r < nrows && j16 == 0) {
      s_m[r] = M;
      s_z[r] = S;
    }
  }

  __syncthreads();
  if (tid < 64) {
    bool reject = false;
    float p = NAN, q = NAN, ua = NAN;
    if (lane < G) {
      p = expf(tv - s_m[lane]) / s_z[lane];
      q = expf(dv - s_m[G + 1 + lane]) / s_z[G + 1 + lane];
      ua = a.uniforms ? a.uniforms[((size_t)b * (G + 1) + lane) * 2 + 0] : philox_uniform(a.seed, a.offset, b, lane, 0);
      reject = !(ua * q < p);
    }
    const uint64_t rm = __ballot(reject);
    const int jstar = rm ? (__ffsll((long long)rm) - 1) : G;
    const float us = a.uniforms ? a.uniforms[((size_t)b * (G + 1) + jstar) * 2 + 1]
                                : philox_uniform(a.seed, a.offset, b, jstar, 1);
    if (lane == 0) {
      *s_jstar = jstar;
      *s_us = us;
    }
    if (write_diag && a.diag && lane <= G) {
      float* dg = a.diag + ((size_t)b * (G + 1) + lane) * 4;
      const bool used = lane <= jstar && lane < G;
      dg[0] = used ? p : NAN;
      dg[1] = used ? q : NAN;
      dg[2] = used ? ua : NAN;
      dg[3] = lane == jstar ? us : NAN;
    }
  }
  __syncthreads();
}

// Uniform of stream `st` (0 = accept test, 1 = sample) at position j.
__device__ __forceinline__ float verify_uniform(const VerifyArgs& a, int b, int j, int st) {
  return a.uniforms ? a.uniforms[((size_t)b * (a.G + 1) + j) * 2 + st] : philox_uniform(a.seed, a.offset, b, j, st);
}

__device__ __forceinline__ RowWeights sampled_row(const VerifyArgs& a, int b, int jstar, const float* s_m,
                                                  const float* s_z) {
  RowWeights rw;
  rw.t = a.tl + ((size_t)b * (a.G + 1) + jstar) * a.V;
  rw.ot = row_offset(s_m[jstar], s_z[jstar]);
  rw.d = nullptr;
  rw.od = 0.f;
  if (jstar < a.G) {
    rw.d = a.dl + ((size_t)b * a.G + jstar) * a.V;
    rw.od = row_offset(s_m[a.G + 1 + jstar], s_z[a.G + 1 + jstar]);
  }
  return rw;
}

// Tile masses (wave inclusive-scan totals) of tiles [t0, t1) of a row into
// s_tile[0 .. t1-t0), and into g_tile[0 .. t1-t0) when it is given.  Tiles go
// round-robin to the waves; each wave issues the loads of up to TPW tiles
// before weighting any of them.  The weights and sums are the same for every
// TPW and NT.
template <int TPW, bool NT>
__device__ void tile_masses(const RowWeights& rw, int V, bool vec, int t0, int t1, float* s_tile,
                            float* g_tile = nullptr) {
  constexpr int kTilesPerWave = TPW;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  for (int tb = t0; tb < t1; tb += nw * kTilesPerWave) {
    float4 tv[kTilesPerWave], dv[kTilesPerWave];
#pragma unroll
    for (int i = 0; i < kTilesPerWave; ++i) {
      const int t = tb + wave + i * nw;
      const int e = t * kTile + lane * 4;
      tv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      dv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < t1) {
        tv[i] = load4<NT>(rw.t, e, V, vec);
        if (rw.d) dv[i] = load4<NT>(rw.d, e, V, vec);
      }
    }
#pragma unroll
    for (int i = 0; i < kTilesPerWave; ++i) {
      const int t = tb + wave + i * nw;
      if (t >= t1) continue;   // wave-uniform
      float wv[4];
      weights4(rw, tv[i], dv[i], t * kTile + lane * 4, V, wv);
      const float incl = wave_incl_scan(((wv[0] + wv[1]) + wv[2]) + wv[3]);
      if (lane == 63) {
        s_tile[t - t0] = incl;
        if (g_tile) g_tile[t - t0] = incl;
      }
    }
  }
}

// First index in [0, n) whose running sum of v[] exceeds x, computed by one
// wave (lanes own contiguous index ranges; fixed order).  Returns the running
// sum before it in *before.  If rounding leaves x at or beyond the total,
// returns the last index with v > 0 and *before = +inf (-1 if none).
__device__ int wave_first_crossing(const float* v, int n, float x, float* before) {
  const int lane = threadIdx.x & 63;
  const int per = (n + 63) / 64;
  const int i0 = min(lane * per, n), i1 = min(i0 + per, n);
  float sum = 0.f;
  int last_pos = -1;
  for (int i = i0; i < i1; ++i) {
    sum += v[i];
    if (v[i] > 0.f) last_pos = i;
  }
  const float incl = wave_incl_scan(sum);
  float run = incl - sum;
  int pick = -1;
  float pick_before = 0.f;
  for (int i = i0; i < i1; ++i) {
    if (pick < 0 && run + v[i] > x) {
      pick = i;
      pick_before = run;
    }
    run += v[i];
  }
  const uint64_t found = __ballot(pick >= 0);
  if (found) {
    const int src = __ffsll((long long)found) - 1;
    *before = __shfl(pick_before, src, 64);
    return __shfl(pick, src, 64);
  }
  const uint64_t has = __ballot(last_pos >= 0);
  *before = INFINITY;
  return has ? __shfl(last_pos, 63 - __clzll((long long)has), 64) : -1;
}

// Early-exit verification, one launch per position j = 0..P-1, then one
// launch for the rest (positions P..G; P = kPhasedPositions, or G when the
// chain is shorter).  The protocol stops at the first rejection, so a
// sequence's rows past it are not read, while the few chains still accepted
// after P positions read their remaining rows in one pass.  Grid (chunk,
// sequence, row) over the rows of positions j..jl: target rows j..jl, then
// draft rows j..min(jl, G-1).  Wave 0 of every workgroup first runs the
// accept test of position j - 1 from the previous launch's partials (all
// workgroups of a sequence get the same bits; a chain that stopped earlier
// skips the arithmetic).  Workgroups of a chain that is no longer accepted
// exit; the others fold their chunk into (max, sum) as the stats pass does,
// and (for a single position) the one whose chunk holds drafted token j
// records its logit for the next launch's test.  The chunk-0 workgroup of
// the first row records the outcome (reach flag, diagnostics, and the
// decision record on a rejection).  The mass kernel decides positions P..G.
template <bool NT>
__global__ __launch_bounds__(kStatThreads) void verify_phase_kernel(VerifyArgs a, VerifyWs ws, int j, int jl) {
  __shared__ float2 s_w[kStatThreads / 64];
  __shared__ int s_go;
  const int c = blockIdx.x;
  const int b = blockIdx.y;
  const int which = blockIdx.z;
  const int G = a.G, B = a.B;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int ntr = jl - j + 1;   // target rows of the launch
  const int r = which < ntr ? j + which : G + 1 + j + (which - ntr);
  const float* row = row_ptr(a, b, r);
  const int e0 = c * a.chunk;
  const int e1 = min(e0 + a.chunk, a.V);
  const bool lead = c == 0 && which == 0;
  const bool single = jl == j;   // one position: record the drafted token's logit
  const float4 ninf = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
  // a batch of the chunk's logits (clamped inside it, masked when used)
  auto load_batch = [&](int e, float4 (&x)[kPhaseU]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kPhaseU; ++u) {
      const int ee = e + u * kStatStep;
      if (a.vec) {
        const float4 v = ld16<NT>(row + (min(ee, e1 - 1) & ~3));
        x[u] = ee < e1 ? v : ninf;
      } else {
        x[u] = ee < e1 ? load4(row, ee, e1, false) : ninf;
      }
    }
  };
  float4 x[kPhaseU];
  const int eb = e0 + tid * 4;
  const int dj = single && j < G ? min(max(a.drafts[(size_t)b * G + j], 0), a.V - 1) : 0;
  if (tid < 64) {
    bool go = true;
    if (j > 0) {
      const int jp = j - 1;
      // every load of the test is issued together with the reach flag (all
      // addresses are valid whatever it says)
      const bool reached = ws.reach[(size_t)jp * B + b] != 0;
      const float tv = ws.dlog[((size_t)b * G + jp) * 2 + 0];
      const float dv = ws.dlog[((size_t)b * G + jp) * 2 + 1];
      const float2* pt = a.part + ((size_t)b * (2 * G + 1) + (lane < 16 ? jp : G + 1 + jp)) * a.nchunks;
      float2 pv[kPhaseFoldMax];
#pragma unroll
      for (int k = 0; k < kPhaseFoldMax; ++k) pv[k] = pt[min((lane & 15) + 16 * k, a.nchunks - 1)];
      const float ua_in = a.uniforms ? a.uniforms[((size_t)b * (G + 1) + jp) * 2] : 0.f;
      bool accept = false;
      float M = -INFINITY, S = 0.f, Md = -INFINITY, Sd = 0.f, p = NAN, q = NAN, ua = NAN;
      if (reached) {   // wave-uniform: a stopped chain skips the arithmetic
        // lanes 0-15 fold the target row, the others the draft row, in the
        // order of decide() (the same bits)
#pragma unroll
        for (int k = 0; k < kPhaseFoldMax; ++k)
          if ((lane & 15) + 16 * k < a.nchunks) ms_merge(M, S, pv[k].x, pv[k].y);
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) {
          const float m2 = __shfl_xor(M, o, 64);
          const float s2 = __shfl_xor(S, o, 64);
          ms_merge(M, S, m2, s2);
        }
        Md = __shfl(M, 16, 64);
        Sd = __shfl(S, 16, 64);
        ua = a.uniforms ? ua_in : philox_uniform(a.seed, a.offset, b, jp, 0);
        p = expf(tv - M) / S;
        q = expf(dv - Md) / Sd;
        accept = ua * q < p;
      }
      go = reached && accept;
      if (lead && lane == 0) {
        ws.reach[(size_t)j * B + b] = go ? 1 : 0;
        float us = NAN;
        if (reached && !accept) {
          Decision dd;
          dd.jstar = jp;
          dd.us = us = verify_uniform(a, b, jp, 1);
          dd.ot = row_offset(M, S);
          dd.od = row_offset(Md, Sd);
          dd.pad0 = dd.pad1 = dd.pad2 = dd.pad3 = 0;
          ws.dec[b] = dd;
        }
        if (a.diag) {
          float* dg = a.diag + ((size_t)b * (G + 1) + jp) * 4;
          dg[0] = reached ? p : NAN;
          dg[1] = reached ? q : NAN;
          dg[2] = reached ? ua : NAN;
          dg[3] = us;
        }
      }
    } else if (lead && lane == 0) {
      ws.reach[b] = 1;
    }
    if (lane == 0) s_go = go ? 1 : 0;
  }
  __syncthreads();
  if (!s_go) return;
  load_batch(eb, x);
  if (single && j < G && tid == 0 && dj >= e0 && dj < e1) ws.dlog[((size_t)b * G + j) * 2 + which] = row[dj];
  float m = -INFINITY, s = 0.f;
  for (int e = eb;;) {
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kPhaseU; ++u) bm = fmaxf(bm, fmaxf(fmaxf(x[u].x, x[u].y), fmaxf(x[u].z, x[u].w)));
    const float M = fmaxf(m, bm);
    if (M != -INFINITY) {
      const float Mc = M * kLog2e;
      float t = 0.f;
#pragma unroll
      for (int u = 0; u < kPhaseU; ++u) {
        t += fast_exp2(fmaf(x[u].x, kLog2e, -Mc));
        t += fast_exp2(fmaf(x[u].y, kLog2e, -Mc));
        t += fast_exp2(fmaf(x[u].z, kLog2e, -Mc));
        t += fast_exp2(fmaf(x[u].w, kLog2e, -Mc));
      }
      s = s * fast_exp2((m - M) * kLog2e) + t;
      m = M;
    }
    e += kPhaseU * kStatStep;
    if (e >= e1) break;
    load_batch(e, x);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64);
    const float s2 = __shfl_xor(s, o, 64);
    ms_merge(m, s, m2, s2);
  }
  const int wave = tid >> 6;
  if (lane == 0) s_w[wave] = make_float2(m, s);
  __syncthreads();
  if (tid == 0) {
    float M = s_w[0].x, S = s_w[0].y;
    for (int w = 1; w < kStatThreads / 64; ++w) ms_merge(M, S, s_w[w].x, s_w[w].y);
    a.part[((size_t)b * (2 * G + 1) + r) * a.nchunks + c] = make_float2(M, S);
  }
}

// Kernel 2: the decision of each sequence.
__global__ __launch_bounds__(kDecideThreads) void verify_decide_kernel(VerifyArgs a, VerifyWs ws) {
  __shared__ float s_m[2 * kMaxG + 1], s_z[2 * kMaxG + 1];
  __shared__ int s_jstar;
  __shared__ float s_us;
  const int b = blockIdx.x;
  decide(a, ws, b, s_m, s_z, &s_jstar, &s_us, true);
  if (threadIdx.x == 0) {
    const RowWeights rw = sampled_row(a, b, s_jstar, s_m, s_z);
    Decision dd;
    dd.jstar = s_jstar;
    dd.us = s_us;
    dd.ot = rw.ot;
    dd.od = rw.od;
    dd.pad0 = dd.pad1 = dd.pad2 = dd.pad3 = 0;
    ws.dec[b] = dd;
  }
}

// Sampled row of sequence b as its decision record states it.
__device__ __forceinline__ RowWeights decided_row(const VerifyArgs& a, const Decision& dd, int b) {
  RowWeights rw;
  rw.t = a.tl + ((size_t)b * (a.G + 1) + dd.jstar) * a.V;
  rw.ot = dd.ot;
  rw.d = dd.jstar < a.G ? a.dl + ((size_t)b * a.G + dd.jstar) * a.V : nullptr;
  rw.od = dd.od;
  return rw;
}

// How the mass kernel learns the decision of its sequence.
constexpr int kMassRecord = 0;   // the decide kernel's record
constexpr int kMassDecide = 1;   // runs the decision itself (a few sequences)
constexpr int kMassPhased = 2;   // early exit: the launch's record, or the decision of a chain that reached the last launch

// Kernel 3: the mass of one chunk (CT tiles) of the sampled row (sum of its
// tile masses in tile order).  With kMassDecide (a few sequences, where one
// launch costs more than the repeated work) every workgroup runs the
// decision itself from the chunk partials, chunk 0 records it for the pick
// kernel, and the separate decide launch is skipped; the decision is the
// same bits either way.  With kMassPhased, a chain that stopped before the
// last early-exit launch has its record; one that reached it is decided
// here over every position, as with kMassDecide.
template <int CT, bool NT, int MODE>
__global__ __launch_bounds__(kMassThreads) void verify_mass_kernel(VerifyArgs a, VerifyWs ws) {
  __shared__ float s_tile[CT];
  const int c = blockIdx.x;
  const int b = blockIdx.y;
  RowWeights rw;
  if constexpr (MODE == kMassPhased) {
    __shared__ float s_m[2 * kMaxG + 1], s_z[2 * kMaxG + 1];
    __shared__ int s_jstar, s_reached;
    __shared__ float s_us;
    if (threadIdx.x == 0) s_reached = ws.reach[(size_t)ws.tail * a.B + b];
    __syncthreads();
    if (s_reached) {
      // the chain reached the last launch's first position: its decision
      // over every position (the same bits as the per-position tests for
      // the positions those already passed)
      decide(a, ws, b, s_m, s_z, &s_jstar, &s_us, c == 0);
      rw = sampled_row(a, b, s_jstar, s_m, s_z);
      if (c == 0 && threadIdx.x == 0) {
        Decision dd;
        dd.jstar = s_jstar;
        dd.us = s_us;
        dd.ot = rw.ot;
        dd.od = rw.od;
        dd.pad0 = dd.pad1 = dd.pad2 = dd.pad3 = 0;
        ws.dec[b] = dd;
      }
    } else {
      rw = decided_row(a, ws.dec[b], b);
      // positions the chain never reached (the per-position launches covered
      // those before the last launch)
      if (c == 0 && a.diag)
        for (int i = threadIdx.x; i < (a.G + 1 - ws.tail) * 4; i += blockDim.x)
          a.diag[((size_t)b * (a.G + 1) + ws.tail) * 4 + i] = NAN;
    }
  } else if constexpr (MODE == kMassDecide) {
    __shared__ float s_m[2 * kMaxG + 1], s_z[2 * kMaxG + 1];
    __shared__ int s_jstar;
    __shared__ float s_us;
    decide(a, ws, b, s_m, s_z, &s_jstar, &s_us, c == 0);
    rw = sampled_row(a, b, s_jstar, s_m, s_z);
    if (c == 0 && threadIdx.x == 0) {
      Decision dd;
      dd.jstar = s_jstar;
      dd.us = s_us;
      dd.ot = rw.ot;
      dd.od = rw.od;
      dd.pad0 = dd.pad1 = dd.pad2 = dd.pad3 = 0;
      ws.dec[b] = dd;
    }
  } else {
    rw = decided_row(a, ws.dec[b], b);
  }
  const int ntiles = (a.V + kTile - 1) / kTile;
  const int t0 = c * CT;
  const int t1 = min(t0 + CT, ntiles);
  constexpr int kTpw = CT / (kMassThreads / 64);
  tile_masses<kTpw, NT>(rw, a.V, a.vec, t0, t1, s_tile, ws.tmass + (size_t)b * ws.ntiles + t0);
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = 0.f;
    for (int t = 0; t < t1 - t0; ++t) m += s_tile[t];
    ws.cmass[(size_t)b * ws.nmass + c] = m;
  }
}

// Kernel 4: one workgroup per sequence picks the emitted token: chunk by the
// chunk masses, tile by the chunk's tile masses, token by a rescan of the
// tile.  Writes emitted tokens and accepted lengths.
template <bool NT>
__global__ __launch_bounds__(kPickThreads) void verify_pick_kernel(VerifyArgs a, VerifyWs ws) {
  __shared__ float s_tile[kMaxTiles];
  __shared__ float s_cm[kMaxMassChunks];
  __shared__ int s_tile_pick;
  __shared__ float s_x;
  __shared__ float s_W;
  __shared__ int s_token;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int G = a.G, V = a.V;
  const Decision dd = ws.dec[b];
  const int jstar = dd.jstar;
  RowWeights rw = decided_row(a, dd, b);
  const int ntiles = (V + kTile - 1) / kTile;
  const int nmass = ws.nmass;
  const int ct = ws.chunk_tiles;
  for (int i = tid; i < nmass; i += kPickThreads) s_cm[i] = ws.cmass[(size_t)b * nmass + i];
  __syncthreads();
  // total mass and the chunk holding u * W (wave 0)
  if (tid < 64) {
    float sum = 0.f;
    for (int i = lane; i < nmass; i += 64) sum += s_cm[i];
    sum = wave_sum(sum);
    float before;
    const int c = wave_first_crossing(s_cm, nmass, dd.us * sum, &before);
    if (lane == 0) {
      s_W = sum;
      s_tile_pick = c < 0 ? 0 : c;
      // no crossing (rounding put u * W at or past the scanned total): +inf
      // makes the tile and token levels take their last positive entry too
      s_x = before == INFINITY ? INFINITY : dd.us * sum - before;
    }
  }
  __syncthreads();
  int t0, t1;
  bool full_row = false;
  if (s_W > 0.f || rw.d == nullptr) {
    t0 = s_tile_pick * ct;
    t1 = min(t0 + ct, ntiles);
  } else {
    // residual without mass (reachable only through rounding): draw from p
    rw.d = nullptr;
    t0 = 0;
    t1 = ntiles;
    full_row = true;
  }
  float x = s_x;
  __syncthreads();
  if (full_row) {
    tile_masses<4, NT>(rw, V, a.vec, t0, t1, s_tile);
  } else {
    // the mass kernel stored these tile masses (the same bits a rescan gives)
    const float* tm = ws.tmass + (size_t)b * ws.ntiles;
    for (int t = t0 + tid; t < t1; t += kPickThreads) s_tile[t - t0] = tm[t];
  }
  __syncthreads();
  if (tid < 64) {
    if (full_row) {
      float sum = 0.f;
      for (int i = lane; i < t1 - t0; i += 64) sum += s_tile[i];
      x = dd.us * wave_sum(sum);
    }
    float before;
    const int t = wave_first_crossing(s_tile, t1 - t0, x, &before);
    if (lane == 0) {
      s_tile_pick = t < 0 ? -1 : t0 + t;
      s_x = before == INFINITY ? INFINITY : x - before;
    }
  }
  __syncthreads();
  // token inside the picked tile (wave 0)
  if (tid < 64) {
    const int tp = s_tile_pick;
    int token = -1;
    if (tp >= 0) {
      float wv[4], incl;
      const int e = tp * kTile + lane * 4;
      tile_weights(rw, e, V, a.vec, wv, incl);
      const float xx = s_x;
      const float lane_sum = ((wv[0] + wv[1]) + wv[2]) + wv[3];
      const float excl = incl - lane_sum;
      int pick = -1;
      if (incl > xx) {
        float run = excl;
        for (int i = 0; i < 4; ++i) {
          run += wv[i];
          if (run > xx && wv[i] > 0.f) {
            pick = e + i;
            break;
          }
        }
        if (pick < 0)
          for (int i = 3; i >= 0; --i)
            if (wv[i] > 0.f) {
              pick = e + i;
              break;
            }
      }
      const uint64_t found = __ballot(pick >= 0);
      if (found) {
        token = __shfl(pick, __ffsll((long long)found) - 1, 64);
      } else {
        int last = -1;
        for (int i = 3; i >= 0; --i)
          if (wv[i] > 0.f) {
            last = e + i;
            break;
          }
        const uint64_t has = __ballot(last >= 0);
        if (has) token = __shfl(last, 63 - __clzll((long long)has), 64);
      }
    }
    if (lane == 0) s_token = token;
  }
  __syncthreads();
  if (tid <= G) {
    int32_t v = -1;
    if (tid < jstar) v = a.drafts[(size_t)b * G + tid];
    else if (tid == jstar) v = s_token;
    a.emitted[(size_t)b * (G + 1) + tid] = v;
  }
  if (tid == 0) a.acc_len[b] = jstar;
}

template <int CT, int MODE>
void launch_mass(bool nt, dim3 grid, hipStream_t s, const VerifyArgs& a, const VerifyWs& ws) {
  if (nt) hipLaunchKernelGGL((verify_mass_kernel<CT, true, MODE>), grid, dim3(kMassThreads), 0, s, a, ws);
  else hipLaunchKernelGGL((verify_mass_kernel<CT, false, MODE>), grid, dim3(kMassThreads), 0, s, a, ws);
}

template <int MODE>
void launch_mass_ct(int ct, bool nt, dim3 grid, hipStream_t s, const VerifyArgs& a, const VerifyWs& ws) {
  if (ct == kBigChunkTiles) launch_mass<kBigChunkTiles, MODE>(nt, grid, s, a, ws);
  else launch_mass<kSmallChunkTiles, MODE>(nt, grid, s, a, ws);
}

// Logits per stats workgroup: whole rows when the rows alone give about
// kStatTargetWgs workgroups, else rows split into chunks of whole load
// rounds so that about that many run.
int chunk_for_rows(int64_t rows, int V, int step, int target = kStatTargetWgs, int64_t max_chunks = 1 << 30) {
  const int64_t steps = (V + step - 1) / step;
  int64_t want = (target + rows - 1) / rows;   // chunks per row
  want = want < 1 ? 1 : want > steps ? steps : want;
  want = want > max_chunks ? max_chunks : want;
  return (int)((steps + want - 1) / want) * step;
}

// Tiles per residual-mass chunk: 8K-logit chunks (kBigChunkTiles tiles)
// when there are enough sequences to fill the GPU with them, else 4K.
int mass_chunk_tiles(int B, int V) {
  const int64_t big = (V + kBigChunkTiles * kTile - 1) / (kBigChunkTiles * kTile);
  return (int64_t)B * big >= 1024 ? kBigChunkTiles : kSmallChunkTiles;
}

// The schedule: early exit from kPhasedMinBytes of logits on.  The
// environment variable DSA_VERIFY_SCHEDULE = "phased" or "onepass" overrides
// the size rule (both give the same decisions; for tests and tuning).
bool phased_mode(int B, int G, int V) {
  const char* e = getenv("DSA_VERIFY_SCHEDULE");
  if (e && strcmp(e, "phased") == 0) return true;
  if (e && strcmp(e, "onepass") == 0) return false;
  return (double)B * (2 * G + 1) * V * sizeof(float) >= (double)kPhasedMinBytes;
}

// Logits per stats workgroup: the one-pass stats cover all 2G+1 rows at
// once; a phase covers two rows per sequence.
int stats_chunk(int B, int G, int V, bool phased) {
  return phased ? chunk_for_rows((int64_t)B * 2, V, kStatStep, kPhaseTargetWgs, 16 * kPhaseFoldMax)
                : chunk_for_rows((int64_t)B * (2 * G + 1), V, kStatStep);
}

// Workspace layout for the schedule `phased`; its size covers both
// schedules, so that the size query does not depend on the choice.
size_t verify_ws(int B, int G, int V, bool phased, int* nchunks, int* chunk, VerifyWs* out, char* base) {
  const int ch = stats_chunk(B, G, V, phased);
  const int nc = (V + ch - 1) / ch;
  const int ch1 = stats_chunk(B, G, V, false), ch2 = stats_chunk(B, G, V, true);
  const int nc_max = max((V + ch1 - 1) / ch1, (V + ch2 - 1) / ch2);
  const int ct = mass_chunk_tiles(B, V);
  const int nm = (V + ct * kTile - 1) / (ct * kTile);
  if (nchunks) *nchunks = nc;
  if (chunk) *chunk = ch;
  const size_t part = align_up((size_t)B * (2 * G + 1) * nc_max * sizeof(float2), 256);
  const size_t dec = align_up((size_t)B * sizeof(Decision), 256);
  const size_t cm = align_up((size_t)B * nm * sizeof(float), 256);
  const int nt = (V + kTile - 1) / kTile;
  const size_t tm = align_up((size_t)B * nt * sizeof(float), 256);
  const size_t rc = align_up((size_t)(G + 1) * B * sizeof(int), 256);
  const size_t dl = align_up((size_t)B * G * 2 * sizeof(float), 256);
  if (out) {
    out->part = reinterpret_cast<float2*>(base);
    out->dec = reinterpret_cast<Decision*>(base + part);
    out->cmass = reinterpret_cast<float*>(base + part + dec);
    out->tmass = reinterpret_cast<float*>(base + part + dec + cm);
    out->reach = reinterpret_cast<int*>(base + part + dec + cm + tm);
    out->dlog = reinterpret_cast<float*>(base + part + dec + cm + tm + rc);
    out->nmass = nm;
    out->ntiles = nt;
    out->chunk_tiles = ct;
    out->phased = phased;
  }
  return part + dec + cm + tm + rc + dl;
}

// ---------------------------------------------------------------------------
// Greedy verification: d_j is accepted iff it is the argmax of target row j
// (ties to the lower token id); the first mismatch emits that argmax, and a
// fully accepted chain emits the argmax of the last target row.  Only the
// G+1 target rows are read, once.
// ---------------------------------------------------------------------------
struct ArgMax {
  float v;
  int i;
};

// Larger value wins; equal values go to the lower index.  Associative and
// commutative, so every reduction order gives the same winner.
__device__ __forceinline__ ArgMax am_pick(ArgMax a, ArgMax b) {
  return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}

__device__ __forceinline__ ArgMax am_wave(ArgMax a) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    ArgMax b;
    b.v = __shfl_xor(a.v, o, 64);
    b.i = __shfl_xor(a.i, o, 64);
    a = am_pick(a, b);
  }
  return a;
}

struct GreedyArgs {
  const float* tl;
  const int32_t* drafts;
  int B, G, V, nchunks, chunk;
  int32_t* acc_len;
  int32_t* emitted;
  ArgMax* part;   // [B][G+1][nchunks]
  int* reach;     // early exit: [G+1][B], 1 where the chain reached position j
  bool vec;
};

// (max, argmax) of logits [e0, e1) of a row, reduced over the workgroup;
// the result is valid in thread 0.
template <bool NT>
__device__ ArgMax chunk_argmax(const GreedyArgs& a, const float* row, int e0, int e1) {
  __shared__ ArgMax s_w[kArgThreads / 64];
  ArgMax best{-INFINITY, INT_MAX};
  for (int e = e0 + threadIdx.x * 4; e < e1; e += kArgU * kArgStep) {
    float4 x[kArgU];
#pragma unroll
    for (int u = 0; u < kArgU; ++u) {
      const int ee = e + u * kArgStep;
      if (a.vec) x[u] = ld16<NT>(row + (min(ee, e1 - 1) & ~3));
      else x[u] = load4(row, min(ee, e1 - 1), e1, false);
    }
#pragma unroll
    for (int u = 0; u < kArgU; ++u) {
      const int ee = e + u * kArgStep;   // ascending within the thread: strict > keeps the first
      if (ee + 0 < e1 && x[u].x > best.v) best = ArgMax{x[u].x, ee + 0};
      if (ee + 1 < e1 && x[u].y > best.v) best = ArgMax{x[u].y, ee + 1};
      if (ee + 2 < e1 && x[u].z > best.v) best = ArgMax{x[u].z, ee + 2};
      if (ee + 3 < e1 && x[u].w > best.v) best = ArgMax{x[u].w, ee + 3};
    }
  }
  best = am_wave(best);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) s_w[wave] = best;
  __syncthreads();
  ArgMax r = s_w[0];
  for (int w = 1; w < kArgThreads / 64; ++w) r = am_pick(r, s_w[w]);
  return r;
}

// Kernel 1: (max, argmax) of each chunk of each target row.
template <bool NT>
__global__ __launch_bounds__(kArgThreads) void greedy_argmax_kernel(GreedyArgs a) {
  const int c = blockIdx.x;
  const int rr = blockIdx.y;   // b * (G+1) + j
  const float* row = a.tl + (size_t)rr * a.V;
  const int e0 = c * a.chunk;
  const int e1 = min(e0 + a.chunk, a.V);
  const ArgMax r = chunk_argmax<NT>(a, row, e0, e1);
  if (threadIdx.x == 0) a.part[(size_t)rr * a.nchunks + c] = r;
}

// Winner of the chunk partials of target row j of sequence b (wave 0, all
// lanes; the pick is associative and commutative, so the order is free).  A
// row of -inf only (or NaN, outside the domain) has no winner: token 0.
__device__ __forceinline__ int row_argmax(const GreedyArgs& a, int b, int j) {
  const int lane = threadIdx.x & 63;
  const ArgMax* p = a.part + ((size_t)b * (a.G + 1) + j) * a.nchunks;
  ArgMax best{-INFINITY, INT_MAX};
  for (int c = lane; c < a.nchunks; c += 64) best = am_pick(best, p[c]);
  best = am_wave(best);
  return best.i == INT_MAX ? 0 : best.i;
}

// Emitted tokens and accepted length of a chain stopped at position jstar
// with token `tok` (lanes 0..G of one wave).
__device__ __forceinline__ void greedy_emit(const GreedyArgs& a, int b, int jstar, int tok) {
  const int lane = threadIdx.x & 63;
  if (lane <= a.G) {
    int32_t v = -1;
    if (lane < jstar) v = a.drafts[(size_t)b * a.G + lane];
    else if (lane == jstar) v = tok;
    a.emitted[(size_t)b * (a.G + 1) + lane] = v;
  }
  if (lane == 0) a.acc_len[b] = jstar;
}

// Early-exit greedy verification (large batches): one launch per position
// j = 0..P-1, then one launch over target rows P..G (P =
// kGreedyPhasedPositions, or G for a shorter chain); grid (chunk, sequence,
// row).  Wave 0 of every workgroup first compares draft j - 1 with the
// argmax of target row j - 1 (from the previous launch's partials); the
// chunk-0 workgroup of a chain that stops there emits its tokens.
// Workgroups of chains that stopped exit; the others reduce their chunk of
// target row j + blockIdx.z.  greedy_decide_kernel then decides the chains
// that reached P.
template <bool NT>
__global__ __launch_bounds__(kArgThreads) void greedy_phase_kernel(GreedyArgs a, int j) {
  __shared__ int s_go;
  const int c = blockIdx.x;
  const int b = blockIdx.y;
  const int G = a.G, B = a.B;
  if (threadIdx.x < 64) {
    bool go = true;
    if (j > 0) {
      const int jp = j - 1;
      const bool reached = a.reach[(size_t)jp * B + b] != 0;
      if (reached) {   // wave-uniform
        const int arg = row_argmax(a, b, jp);
        const bool accept = a.drafts[(size_t)b * G + jp] == arg;
        go = accept;
        if (c == 0 && blockIdx.z == 0 && !accept) greedy_emit(a, b, jp, arg);
      } else {
        go = false;
      }
    }
    if (c == 0 && blockIdx.z == 0 && (threadIdx.x & 63) == 0) a.reach[(size_t)j * B + b] = go ? 1 : 0;
    if ((threadIdx.x & 63) == 0) s_go = go ? 1 : 0;
  }
  __syncthreads();
  if (!s_go) return;
  const int jr = j + blockIdx.z;
  const float* row = a.tl + ((size_t)b * (G + 1) + jr) * a.V;
  const int e0 = c * a.chunk;
  const int e1 = min(e0 + a.chunk, a.V);
  const ArgMax r = chunk_argmax<NT>(a, row, e0, e1);
  if (threadIdx.x == 0) a.part[((size_t)b * (G + 1) + jr) * a.nchunks + c] = r;
}

// Kernel 2: one workgroup per sequence folds the chunk winners of its G+1
// rows and compares the drafts with them.
constexpr int kGreedyThreads = 256;

__global__ __launch_bounds__(kGreedyThreads) void greedy_decide_kernel(GreedyArgs a, int from) {
  __shared__ int s_arg[kMaxG + 1];
  const int b = blockIdx.x;
  const int G = a.G;
  // early exit: only the chains that reached position `from` (the others
  // were decided by the per-position launches)
  if (from >= 0 && a.reach[(size_t)from * a.B + b] == 0) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int j = wave; j <= G; j += kGreedyThreads / 64) {
    const ArgMax* p = a.part + ((size_t)b * (G + 1) + j) * a.nchunks;
    ArgMax best{-INFINITY, INT_MAX};
    for (int c = lane; c < a.nchunks; c += 64) best = am_pick(best, p[c]);
    best = am_wave(best);
    // a row of -inf only (or NaN, outside the domain) has no winner: token 0
    if (lane == 0) s_arg[j] = best.i == INT_MAX ? 0 : best.i;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const bool mismatch = lane < G && a.drafts[(size_t)b * G + lane] != s_arg[lane];
    const uint64_t mm = __ballot(mismatch);
    const int jstar = mm ? (__ffsll((long long)mm) - 1) : G;
    if (lane <= G) {
      int32_t v = -1;
      if (lane < jstar) v = a.drafts[(size_t)b * G + lane];
      else if (lane == jstar) v = s_arg[jstar];
      a.emitted[(size_t)b * (G + 1) + lane] = v;
    }
    if (lane == 0) a.acc_len[b] = jstar;
  }
}

// Greedy verification schedule: early exit (one launch per position) from
// kPhasedMinBytes of target logits on, unless DSA_VERIFY_SCHEDULE says
// otherwise (as for spec_verify).
bool greedy_phased(int B, int G, int V) {
  const char* e = getenv("DSA_VERIFY_SCHEDULE");
  if (e && strcmp(e, "phased") == 0) return true;
  if (e && strcmp(e, "onepass") == 0) return false;
  return (double)B * (G + 1) * V * sizeof(float) >= (double)kPhasedMinBytes;
}

// Chunks: the one-pass schedule spreads all G+1 rows of every sequence over
// about kStatTargetWgs workgroups, a phase one row per sequence over about
// kPhaseTargetWgs.  The workspace covers both (its size does not depend on
// the schedule): argmax partials [B][G+1][chunks], then the reach flags.
size_t greedy_ws(int B, int G, int V, bool phased, int* nchunks, int* chunk, int** reach, char* base) {
  const int ch1 = chunk_for_rows((int64_t)B * (G + 1), V, kArgStep);
  const int ch2 = chunk_for_rows((int64_t)B, V, kArgStep, kPhaseTargetWgs);
  const int ch = phased ? ch2 : ch1;
  const int nc_max = max((V + ch1 - 1) / ch1, (V + ch2 - 1) / ch2);
  if (nchunks) *nchunks = (V + ch - 1) / ch;
  if (chunk) *chunk = ch;
  const size_t part = align_up((size_t)B * (G + 1) * nc_max * sizeof(ArgMax), 256);
  if (reach) *reach = reinterpret_cast<int*>(base + part);
  return part + align_up((size_t)(G + 1) * B * sizeof(int), 256);
}

}  // namespace
}  // namespace dsa

extern "C" size_t spec_verify_workspace_size(int B, int G, int V) {
  if (B < 1 || G < 1 || V < 1) return 0;
  return dsa::verify_ws(B, G, V, false, nullptr, nullptr, nullptr, nullptr);
}

extern "C" dsa_status spec_verify(const float* target_logits, const float* draft_logits,
                                  const int32_t* draft_tokens, int B, int G, int V, const float* uniforms,
                                  uint64_t seed, uint64_t offset, int32_t* accepted_len, int32_t* emitted,
                                  float* diag, void* workspace, size_t workspace_bytes, void* stream) {
  using namespace dsa;
  clear_error();
  DSA_REQUIRE(target_logits && draft_logits && draft_tokens && accepted_len && emitted, DSA_ERR_INVALID_ARG,
              "spec_verify: null pointer argument");
  DSA_REQUIRE(B >= 1 && G >= 1 && V >= 1, DSA_ERR_INVALID_ARG, "spec_verify: sizes must be positive (B=%d G=%d V=%d)",
              B, G, V);
  DSA_REQUIRE(G <= kMaxG, DSA_ERR_UNSUPPORTED, "spec_verify: G=%d > %d", G, kMaxG);
  DSA_REQUIRE(V <= kMaxV, DSA_ERR_UNSUPPORTED, "spec_verify: V=%d > %d", V, kMaxV);
  DSA_REQUIRE((int64_t)B * (2 * G + 1) <= 65535, DSA_ERR_UNSUPPORTED, "spec_verify: B*(2G+1)=%lld rows > 65535",
              (long long)B * (2 * G + 1));
  int nchunks = 0, chunk = 0;
  const bool phased = phased_mode(B, G, V);
  const size_t need = verify_ws(B, G, V, phased, &nchunks, &chunk, nullptr, nullptr);
  DSA_REQUIRE(workspace && workspace_bytes >= need, DSA_ERR_WORKSPACE,
              "spec_verify: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  VerifyArgs a{};
  a.tl = target_logits;
  a.dl = draft_logits;
  a.drafts = draft_tokens;
  a.B = B;
  a.G = G;
  a.V = V;
  a.nchunks = nchunks;
  a.chunk = chunk;
  a.uniforms = uniforms;
  a.seed = seed;
  a.offset = offset;
  a.acc_len = accepted_len;
  a.emitted = emitted;
  a.diag = diag;
  VerifyWs ws;
  verify_ws(B, G, V, phased, nullptr, nullptr, &ws, static_cast<char*>(workspace));
  a.part = ws.part;
  a.vec = (V % 4 == 0) && aligned16(target_logits) && aligned16(draft_logits);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool nt = (size_t)B * (2 * G + 1) * V * sizeof(float) > kStreamBytes;
  const dim3 gs(nchunks, B * (2 * G + 1)), gm(ws.nmass, B);
  dsa_status st;
  if (ws.phased) {
    // early exit: one launch per position up to the tail, then the tail's
    // rows in one launch
    ws.tail = min(kPhasedPositions, G);
    for (int j = 0; j <= ws.tail; ++j) {
      const int jl = j < ws.tail ? j : G;
      const int nrows = (jl - j + 1) + (min(jl, G - 1) - j + 1);
      const dim3 gp(nchunks, B, nrows);
      if (nt) hipLaunchKernelGGL(verify_phase_kernel<true>, gp, dim3(kStatThreads), 0, s, a, ws, j, jl);
      else hipLaunchKernelGGL(verify_phase_kernel<false>, gp, dim3(kStatThreads), 0, s, a, ws, j, jl);
      st = launch_status("spec_verify(phase)");
      if (st != DSA_OK) return st;
    }
    launch_mass_ct<kMassPhased>(ws.chunk_tiles, nt, gm, s, a, ws);
    st = launch_status("spec_verify(mass)");
    if (st != DSA_OK) return st;
    if (nt) hipLaunchKernelGGL(verify_pick_kernel<true>, dim3(B), dim3(kPickThreads), 0, s, a, ws);
    else hipLaunchKernelGGL(verify_pick_kernel<false>, dim3(B), dim3(kPickThreads), 0, s, a, ws);
    return launch_status("spec_verify(pick)");
  }
  if (nt) hipLaunchKernelGGL(verify_stats_kernel<true>, gs, dim3(kStatThreads), 0, s, a);
  else hipLaunchKernelGGL(verify_stats_kernel<false>, gs, dim3(kStatThreads), 0, s, a);
  st = launch_status("spec_verify(stats)");
  if (st != DSA_OK) return st;
#ifndef DSA_VERIFY_FUSE_MAX_B
#define DSA_VERIFY_FUSE_MAX_B 16
#endif
  // up to DSA_VERIFY_FUSE_MAX_B sequences the decision runs inside the mass
  // kernel (three launches); beyond, in a kernel of its own
  const bool fuse = B <= DSA_VERIFY_FUSE_MAX_B;
  if (!fuse) {
    hipLaunchKernelGGL(verify_decide_kernel, dim3(B), dim3(kDecideThreads), 0, s, a, ws);
    st = launch_status("spec_verify(decide)");
    if (st != DSA_OK) return st;
  }
  if (fuse) launch_mass_ct<kMassDecide>(ws.chunk_tiles, nt, gm, s, a, ws);
  else launch_mass_ct<kMassRecord>(ws.chunk_tiles, nt, gm, s, a, ws);
  st = launch_status("spec_verify(mass)");
  if (st != DSA_OK) return st;
  if (nt) hipLaunchKernelGGL(verify_pick_kernel<true>, dim3(B), dim3(kPickThreads), 0, s, a, ws);
  else hipLaunchKernelGGL(verify_pick_kernel<false>, dim3(B), dim3(kPickThreads), 0, s, a, ws);
  return launch_status("spec_verify(pick)");
}

extern "C" size_t spec_verify_greedy_workspace_size(int B, int G, int V) {
  if (B < 1 || G < 1 || V < 1) return 0;
  return dsa::greedy_ws(B, G, V, false, nullptr, nullptr, nullptr, nullptr);
}

extern "C" dsa_status spec_verify_greedy(const float* target_logits, const int32_t* draft_tokens, int B, int G,
                                         int V, int32_t* accepted_len, int32_t* emitted, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  using namespace dsa;
  clear_error();
  DSA_REQUIRE(target_logits && draft_tokens && accepted_len && emitted, DSA_ERR_INVALID_ARG,
              "spec_verify_greedy: null pointer argument");
  DSA_REQUIRE(B >= 1 && G >= 1 && V >= 1, DSA_ERR_INVALID_ARG,
              "spec_verify_greedy: sizes must be positive (B=%d G=%d V=%d)", B, G, V);
  DSA_REQUIRE(G <= kMaxG, DSA_ERR_UNSUPPORTED, "spec_verify_greedy: G=%d > %d", G, kMaxG);
  DSA_REQUIRE(V <= kMaxV, DSA_ERR_UNSUPPORTED, "spec_verify_greedy: V=%d > %d", V, kMaxV);
  DSA_REQUIRE((int64_t)B * (G + 1) <= 65535, DSA_ERR_UNSUPPORTED, "spec_verify_greedy: B*(G+1)=%lld rows > 65535",
              (long long)B * (G + 1));
  int nchunks = 0, chunk = 0;
  int* reach = nullptr;
  const bool phased = greedy_phased(B, G, V);
  const size_t need = greedy_ws(B, G, V, phased, &nchunks, &chunk, nullptr, nullptr);
  DSA_REQUIRE(workspace && workspace_bytes >= need, DSA_ERR_WORKSPACE,
              "spec_verify_greedy: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  greedy_ws(B, G, V, phased, nullptr, nullptr, &reach, static_cast<char*>(workspace));
  GreedyArgs a{};
  a.tl = target_logits;
  a.drafts = draft_tokens;
  a.B = B;
  a.G = G;
  a.V = V;
  a.nchunks = nchunks;
  a.chunk = chunk;
  a.acc_len = accepted_len;
  a.emitted = emitted;
  a.part = static_cast<ArgMax*>(workspace);
  a.reach = reach;
  a.vec = (V % 4 == 0) && aligned16(target_logits);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool nt = (size_t)B * (G + 1) * V * sizeof(float) > kStreamBytes;
  if (phased) {
    // early exit: positions 0..P-1 one launch each, rows P..G in one, then
    // the decision of the chains that reached P
    const int P = min(kGreedyPhasedPositions, G);
    for (int j = 0; j <= P; ++j) {
      const dim3 gp(nchunks, B, j < P ? 1 : G - P + 1);
      if (nt) hipLaunchKernelGGL(greedy_phase_kernel<true>, gp, dim3(kArgThreads), 0, s, a, j);
      else hipLaunchKernelGGL(greedy_phase_kernel<false>, gp, dim3(kArgThreads), 0, s, a, j);
      const dsa_status st = launch_status("spec_verify_greedy(phase)");
      if (st != DSA_OK) return st;
    }
    hipLaunchKernelGGL(greedy_decide_kernel, dim3(B), dim3(kGreedyThreads), 0, s, a, P);
    return launch_status("spec_verify_greedy(decide)");
  }
  const dim3 g1(nchunks, B * (G + 1));
  if (nt)
    hipLaunchKernelGGL(greedy_argmax_kernel<true>, g1, dim3(kArgThreads), 0, s, a);
  else
    hipLaunchKernelGGL(greedy_argmax_kernel<false>, g1, dim3(kArgThreads), 0, s, a);
  const dsa_status st = launch_status("spec_verify_greedy(argmax)");
  if (st != DSA_OK) return st;
  hipLaunchKernelGGL(greedy_decide_kernel, dim3(B), dim3(kGreedyThreads), 0, s, a, -1);
  return launch_status("spec_verify_greedy(decide)");
}
