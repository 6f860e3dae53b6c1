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
// Two launches, both streaming logits once with 16-byte loads:
//   stats   grid (chunk, row): per 16K-logit chunk of each of the 2G+1 rows of
//           a sequence, the running max and sum of exp(x - max) (fp32,
//           wavefront reductions); partials land in the workspace.
//   decide  one workgroup per sequence: folds the chunk partials in chunk
//           order, tests the G drafts in parallel lanes (first rejection by
//           ballot), then draws from the residual (or bonus) row by inverse
//           CDF: per-256-logit tile masses from a wave inclusive scan, a scan
//           over the tile masses, and a rescan of the one tile that holds the
//           crossing point.
// Uniforms come from the caller or from Philox4x64-10 (Salmon, Moraes, Dror,
// Shaw, SC'11) evaluated in-kernel at counter (offset, b, j, stream).
#include "dsa_common.h"

namespace dsa {
namespace {

constexpr int kStatThreads = 256;
constexpr int kChunk = 16384;        // logits per stats workgroup
constexpr int kDecThreads = 512;
constexpr int kDecWaves = kDecThreads / 64;
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

__device__ __forceinline__ float4 load4(const float* row, int e, int V, bool vec) {
  if (vec && e + 3 < V) return *reinterpret_cast<const float4*>(row + e);
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
  int B, G, V, nchunks;
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

__global__ __launch_bounds__(kStatThreads) void verify_stats_kernel(VerifyArgs a) {
  __shared__ float2 s_w[kStatThreads / 64];
  const int c = blockIdx.x;
  const int rr = blockIdx.y;                 // b * (2G+1) + r
  const int nrows = 2 * a.G + 1;
  const int b = rr / nrows;
  const int r = rr % nrows;
  const float* row = row_ptr(a, b, r);
  const int e0 = c * kChunk;
  const int e1 = min(e0 + kChunk, a.V);
  float m = -INFINITY, s = 0.f;
  for (int e = e0 + threadIdx.x * 4; e < e1; e += kStatThreads * 4) {
    const float4 x = load4(row, e, e1, a.vec);
    const float m4 = fmaxf(fmaxf(x.x, x.y), fmaxf(x.z, x.w));
    const float M = fmaxf(m, m4);
    if (M == -INFINITY) continue;   // nothing but -inf logits so far
    const float ML = M * kLog2e;
    float t = s * fast_exp2(m * kLog2e - ML);
    t += fast_exp2(x.x * kLog2e - ML);
    t += fast_exp2(x.y * kLog2e - ML);
    t += fast_exp2(x.z * kLog2e - ML);
    t += fast_exp2(x.w * kLog2e - ML);
    s = t;
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

// Weight of logit e of the sampled row (0 beyond V).
struct RowWeights {
  const float* t;   // target row
  const float* d;   // draft row (residual) or nullptr (plain softmax of t)
  float mt, inv_zt, md, inv_zd;
  __device__ __forceinline__ float w(float tv, float dv) const {
    const float p = __expf(tv - mt) * inv_zt;
    if (!d) return p;
    const float q = __expf(dv - md) * inv_zd;
    return fmaxf(p - q, 0.f);
  }
};

// Per-lane weights of 4 consecutive logits and their wave inclusive scan.
__device__ __forceinline__ void tile_weights(const RowWeights& rw, int e, int V, bool vec, float wv[4],
                                             float& lane_incl) {
  const float4 tv = load4(rw.t, e, V, vec);
  float4 dv = make_float4(0.f, 0.f, 0.f, 0.f);
  if (rw.d) dv = load4(rw.d, e, V, vec);
  wv[0] = e + 0 < V ? rw.w(tv.x, dv.x) : 0.f;
  wv[1] = e + 1 < V ? rw.w(tv.y, dv.y) : 0.f;
  wv[2] = e + 2 < V ? rw.w(tv.z, dv.z) : 0.f;
  wv[3] = e + 3 < V ? rw.w(tv.w, dv.w) : 0.f;
  float v = ((wv[0] + wv[1]) + wv[2]) + wv[3];
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  lane_incl = v;
}

__global__ __launch_bounds__(kDecThreads) void verify_decide_kernel(VerifyArgs a) {
  __shared__ float s_m[2 * kMaxG + 1], s_z[2 * kMaxG + 1];
  __shared__ float s_tile[kMaxTiles];
  __shared__ int s_jstar;
  __shared__ float s_us;
  __shared__ float s_W;
  __shared__ int s_tile_pick;
  __shared__ float s_x;
  __shared__ int s_token;

  const int b = blockIdx.x;
  const int G = a.G, V = a.V;
  const int nrows = 2 * G + 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // 1. fold chunk partials in chunk order
  if (tid < nrows) {
    const float2* p = a.part + ((size_t)b * nrows + tid) * a.nchunks;
    float M = p[0].x, S = p[0].y;
    for (int c = 1; c < a.nchunks; ++c) ms_merge(M, S, p[c].x, p[c].y);
    s_m[tid] = M;
    s_z[tid] = S;
  }
  __syncthreads();

  // 2. accept tests, one lane per draft position
  if (wave == 0) {
    bool reject = false;
    if (lane < G) {
      const int d = a.drafts[(size_t)b * G + lane];
      const float tv = a.tl[((size_t)b * (G + 1) + lane) * V + d];
      const float dv = a.dl[((size_t)b * G + lane) * V + d];
      const float p = expf(tv - s_m[lane]) / s_z[lane];
      const float q = expf(dv - s_m[G + 1 + lane]) / s_z[G + 1 + lane];
      const float ua = a.uniforms ? a.uniforms[((size_t)b * (G + 1) + lane) * 2 + 0]
                                  : philox_uniform(a.seed, a.offset, b, lane, 0);
      reject = !(ua * q < p);
      if (a.diag) {
        float* dg = a.diag + ((size_t)b * (G + 1) + lane) * 4;
        dg[0] = p;
        dg[1] = q;
        dg[2] = ua;
      }
    }
    const uint64_t rm = __ballot(reject);
    const int jstar = rm ? (__ffsll((long long)rm) - 1) : G;
    if (lane == 0) {
      s_jstar = jstar;
      s_us = a.uniforms ? a.uniforms[((size_t)b * (G + 1) + jstar) * 2 + 1]
                        : philox_uniform(a.seed, a.offset, b, jstar, 1);
    }
    if (a.diag && lane <= G) {
      float* dg = a.diag + ((size_t)b * (G + 1) + lane) * 4;
      if (lane > jstar || lane == G) {
        dg[0] = NAN;
        dg[1] = NAN;
        dg[2] = NAN;
      }
      dg[3] = lane == jstar ? (a.uniforms ? a.uniforms[((size_t)b * (G + 1) + jstar) * 2 + 1]
                                          : philox_uniform(a.seed, a.offset, b, jstar, 1))
                            : NAN;
    }
  }
  __syncthreads();
  const int jstar = s_jstar;

  // 3. inverse-CDF draw from the residual (or bonus) row
  RowWeights rw;
  rw.t = a.tl + ((size_t)b * (G + 1) + jstar) * V;
  rw.mt = s_m[jstar];
  rw.inv_zt = 1.f / s_z[jstar];
  rw.d = nullptr;
  rw.md = 0.f;
  rw.inv_zd = 0.f;
  if (jstar < G) {
    rw.d = a.dl + ((size_t)b * G + jstar) * V;
    rw.md = s_m[G + 1 + jstar];
    rw.inv_zd = 1.f / s_z[G + 1 + jstar];
  }
  const int ntiles = (V + kTile - 1) / kTile;
  for (int pass = 0; pass < 2; ++pass) {
    for (int t = wave; t < ntiles; t += kDecWaves) {
      float wv[4], incl;
      tile_weights(rw, t * kTile + lane * 4, V, a.vec, wv, incl);
      if (lane == 63) s_tile[t] = incl;
    }
    __syncthreads();
    // scan of tile masses by wave 0, lanes own contiguous tile ranges
    if (wave == 0) {
      const int per = (ntiles + 63) / 64;
      const int t0 = min(lane * per, ntiles);
      const int t1 = min(t0 + per, ntiles);
      float sum = 0.f;
      for (int t = t0; t < t1; ++t) sum += s_tile[t];
      float incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
      }
      const float W = __shfl(incl, 63, 64);
      const float x = s_us * W;
      float run = incl - sum;
      int pick = -1, last_pos = -1;
      float pick_run = 0.f;
      for (int t = t0; t < t1; ++t) {
        const float ts = s_tile[t];
        if (pick < 0 && run + ts > x) {
          pick = t;
          pick_run = run;
        }
        if (ts > 0.f) last_pos = t;
        run += ts;
      }
      const uint64_t found = __ballot(pick >= 0);
      if (found) {
        const int src = __ffsll((long long)found) - 1;
        const int tp = __shfl(pick, src, 64);
        const float pr = __shfl(pick_run, src, 64);
        if (lane == 0) {
          s_tile_pick = tp;
          s_x = x - pr;
        }
      } else {
        // rounding left u*W beyond the last cumulative sum: take the last tile with mass
        const uint64_t has = __ballot(last_pos >= 0);
        const int src = has ? 63 - __clzll((long long)has) : 0;
        const int tp = __shfl(last_pos, src, 64);
        if (lane == 0) {
          s_tile_pick = tp;
          s_x = INFINITY;
        }
      }
      if (lane == 0) s_W = W;
    }
    __syncthreads();
    if (s_W > 0.f || pass == 1 || rw.d == nullptr) break;
    // residual without mass (only reachable through rounding): draw from p
    rw.d = nullptr;
    __syncthreads();
  }

  // 4. locate the token inside the picked tile
  if (wave == 0) {
    const int tp = s_tile_pick;
    int token = -1;
    if (tp >= 0) {
      float wv[4], incl;
      const int e = tp * kTile + lane * 4;
      tile_weights(rw, e, V, a.vec, wv, incl);
      const float x = s_x;
      const float lane_sum = ((wv[0] + wv[1]) + wv[2]) + wv[3];
      const float excl = incl - lane_sum;
      int pick = -1;
      if (incl > x) {
        float run = excl;
        for (int i = 0; i < 4; ++i) {
          run += wv[i];
          if (run > x && wv[i] > 0.f) {
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

size_t verify_ws(int B, int G, int V, int* nchunks) {
  const int nc = (V + kChunk - 1) / kChunk;
  if (nchunks) *nchunks = nc;
  return align_up((size_t)B * (2 * G + 1) * nc * sizeof(float2), 256);
}

}  // namespace
}  // namespace dsa

extern "C" size_t spec_verify_workspace_size(int B, int G, int V) {
  if (B < 1 || G < 1 || V < 1) return 0;
  return dsa::verify_ws(B, G, V, nullptr);
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
  int nchunks = 0;
  const size_t need = verify_ws(B, G, V, &nchunks);
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
  a.uniforms = uniforms;
  a.seed = seed;
  a.offset = offset;
  a.acc_len = accepted_len;
  a.emitted = emitted;
  a.diag = diag;
  a.part = static_cast<float2*>(workspace);
  a.vec = (V % 4 == 0) && aligned16(target_logits) && aligned16(draft_logits);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(verify_stats_kernel, dim3(nchunks, B * (2 * G + 1)), dim3(kStatThreads), 0, s, a);
  dsa_status st = launch_status("spec_verify(stats)");
  if (st != DSA_OK) return st;
  hipLaunchKernelGGL(verify_decide_kernel, dim3(B), dim3(kDecThreads), 0, s, a);
  return launch_status("spec_verify(decide)");
}
