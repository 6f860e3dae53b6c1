// Top-k selection per (sequence, row) by radix select (gfx950).
//
// DSA glossary entry ("Optimizing speculative decoding", section "IndexShare
// and KVShare"): a top-k selection keeps the most relevant past positions.
// Order: score descending, then position ascending; output ascending, -1 pad.
//
// Scores are mapped to order-preserving 32-bit keys (-0.0 canonicalised to
// +0.0).  The kept set is {key > K*} plus the lowest positions with key == K*,
// where K* is the k-th largest key.  No sort is needed anywhere: the kept
// positions are produced in position order.
//
// Rows whose keys fit in one CU's LDS take one workgroup and one launch (see
// the one-workgroup path below).  Longer rows take four launches; the row is
// split into chunks of 4096 positions (more when a row has over 4096 chunks):
//   1 zero     clear the row's global 14-bit key histogram
//   2 hist     each chunk's histogram of key bits 31..18 in LDS, added into
//              the row's histogram (16,384 bins) and a 128-bin coarse one
//              with integer atomics
//   3 collect  every workgroup finds the threshold bin T of the row (coarse,
//              then fine) and writes its chunk's positions above T and its
//              candidates (key, position) in T as position-ordered lists,
//              with per-chunk counts (ranks from wave prefix scans; no
//              atomics, so list order is position order)
//   4 finish   one workgroup per row: prefix sums of the chunk counts, a
//              radix select on the candidates' 18 low key bits (two 9-bit
//              rounds), ties to the lower position by list order, and the two
//              ascending lists merged by binary search.
// Integer atomics only (histogram counts, order-free): runs are bitwise
// identical.
#include "dsa_common.h"

namespace dsa {
namespace {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Exclusive prefix of the lanes below this one in a 64-bit ballot mask.
__device__ __forceinline__ uint32_t mask_rank(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

constexpr int kMaxK = 8192;

// ---------------------------------------------------------------------------
// Multi-workgroup pipeline
// ---------------------------------------------------------------------------
constexpr int kDigitBits = 14;                    // first digit: key bits 31..18
constexpr int kLowBits = 32 - kDigitBits;         // resolved among the candidates
constexpr uint32_t kLowMask = (1u << kLowBits) - 1u;
constexpr int kFine = 1 << kDigitBits;            // 16,384 bins
constexpr int kCoarse = 128;
constexpr int kPerCoarse = kFine / kCoarse;       // 128 fine bins per coarse bin
constexpr int kPassThreads = 256;
constexpr int kPassWaves = kPassThreads / 64;
constexpr int kBlock = 4096;                      // positions per load round of a pass workgroup
constexpr int kQuads = kBlock / (4 * kPassThreads);   // four 16-byte loads per thread
#ifndef DSA_TOPK_FIN_THREADS
#define DSA_TOPK_FIN_THREADS 1024
#endif
constexpr int kFinThreads = DSA_TOPK_FIN_THREADS;
constexpr int kMaxChunks = 4 * kFinThreads;       // the finish's prefix sums take 4 chunks per thread
constexpr int kFinWaves = kFinThreads / 64;
constexpr int kCandLds = 4096;                    // candidates resolved in LDS (more: from the workspace)
constexpr int kRadix = 9;                         // two rounds over the 18 low bits
static_assert(2 * kRadix == kLowBits, "two radix rounds cover the low bits");
static_assert(kQuads * 4 * kPassThreads == kBlock, "a load round covers a block");
static_assert(kPerCoarse == kCoarse, "one 128-bin search finds the coarse bin, a second the fine bin in it");

struct PipeWs {
  uint32_t* fine;     // [rows][kFine]
  uint32_t* coarse;   // [rows][kCoarse]
  uint2* counts;      // [rows][chunks]: (above T, in T)
  int32_t* sel;       // [rows][chunks][chunk]: positions above T, ascending
  uint2* cand;        // [rows][chunks][chunk]: (key, position) in T, ascending
  int chunk;          // positions per chunk: kBlock << s
  int chunks;
};

inline int chunk_for(int64_t ld) {
  int64_t c = kBlock;
  while ((ld + c - 1) / c > kMaxChunks) c *= 2;
  return (int)c;
}

inline size_t ws_bytes(int rows, int64_t ld, PipeWs* out, char* base) {
  const int chunk = chunk_for(ld);
  const int chunks = (int)((ld + chunk - 1) / chunk);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  const size_t per = (size_t)chunks * chunk;
  size_t f = take((size_t)rows * kFine * 4);
  size_t c = take((size_t)rows * kCoarse * 4);
  size_t n = take((size_t)rows * chunks * 8);
  size_t sl = take((size_t)rows * per * 4);
  size_t cd = take((size_t)rows * per * 8);
  if (out) {
    out->fine = reinterpret_cast<uint32_t*>(base + f);
    out->coarse = reinterpret_cast<uint32_t*>(base + c);
    out->counts = reinterpret_cast<uint2*>(base + n);
    out->sel = reinterpret_cast<int32_t*>(base + sl);
    out->cand = reinterpret_cast<uint2*>(base + cd);
    out->chunk = chunk;
    out->chunks = chunks;
  }
  return off;
}

// Clears each row's histograms; grid (kZeroParts, rows): each workgroup
// clears 1/kZeroParts of a row's fine bins with one 16-byte store per thread
// (one workgroup per row measured 4-5 us for 16 rows).
constexpr int kZeroParts = kFine / 4 / kPassThreads;
static_assert(kZeroParts * kPassThreads * 4 == kFine, "one 16-byte store per thread");
__global__ __launch_bounds__(kPassThreads) void topk_zero_kernel(PipeWs ws) {
  const int part = blockIdx.x;
  const int row = blockIdx.y;
  reinterpret_cast<uint4*>(ws.fine + (size_t)row * kFine)[part * kPassThreads + threadIdx.x] =
      make_uint4(0u, 0u, 0u, 0u);
  if (part == 0 && threadIdx.x < kCoarse / 4)
    reinterpret_cast<uint4*>(ws.coarse + (size_t)row * kCoarse)[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
}

// Keys of positions p..p+3 (p a multiple of 4).  vec: the row is 16-byte
// aligned and ld a multiple of 4, so one 16-byte load (clamped inside the
// row) serves them; positions at or past L read a clamped copy and are masked
// by the caller.
__device__ __forceinline__ uint4 load_keys4(const float* __restrict__ s, bool vec, int p, int L) {
  float4 v;
  if (vec) {
    v = *reinterpret_cast<const float4*>(s + min(p, (L - 1) & ~3));
  } else {
    v.x = s[min(p, L - 1)];
    v.y = s[min(p + 1, L - 1)];
    v.z = s[min(p + 2, L - 1)];
    v.w = s[min(p + 3, L - 1)];
  }
  return make_uint4(order_key(v.x), order_key(v.y), order_key(v.z), order_key(v.w));
}

__device__ __forceinline__ uint32_t q_at(const uint4& q, int e) {
  return e == 0 ? q.x : e == 1 ? q.y : e == 2 ? q.z : q.w;
}

__global__ __launch_bounds__(kPassThreads) void topk_hist_kernel(const float* __restrict__ scores,
                                                                 const int32_t* __restrict__ row_len, int64_t ld,
                                                                 int k, int vec, PipeWs ws) {
  __shared__ __align__(16) uint32_t h[kFine];
  const int row = blockIdx.y;
  const int tid = threadIdx.x;
  const int L = (int)min((int64_t)row_len[row], ld);   // row_len <= ld is a precondition
  const int64_t c0 = (int64_t)blockIdx.x * ws.chunk;
  if (L <= k || c0 >= L) return;
  const int t_end = (int)min(c0 + ws.chunk, (int64_t)L);
  for (int i = tid; i < kFine / 4; i += kPassThreads) reinterpret_cast<uint4*>(h)[i] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  const float* s = scores + (size_t)row * ld;
  for (int64_t bb = c0; bb < t_end; bb += kBlock) {   // 64-bit: bb + kBlock may pass 2^31 - 1
    const int b = (int)bb;
    uint4 kq[kQuads];
#pragma unroll
    for (int u = 0; u < kQuads; ++u) kq[u] = load_keys4(s, vec != 0, b + (u * kPassThreads + tid) * 4, L);
#pragma unroll
    for (int u = 0; u < kQuads; ++u) {
      const int p = b + (u * kPassThreads + tid) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (p + e < t_end) atomicAdd(&h[q_at(kq[u], e) >> kLowBits], 1u);
    }
  }
  __syncthreads();
  // bins go out lane-consecutively (bin j*256 + t), so a wave's atomics fall
  // on two cache lines per step and merge into few memory-side requests;
  // empty bins are skipped.  All LDS reads are issued before the atomics.
  uint32_t* gf = ws.fine + (size_t)row * kFine;
  constexpr int kPer = kFine / kPassThreads;   // 64
  uint32_t c[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) c[j] = h[j * kPassThreads + tid];
  // coarse bin t/2 gets bins [64t, 64t + 64) of thread t and its neighbour;
  // reads rotated by t so the lanes of a wave hit distinct banks
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) sum += h[tid * kPer + ((j + tid) & (kPer - 1))];
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (c[j]) atomicAdd(gf + j * kPassThreads + tid, c[j]);
  sum += (uint32_t)__shfl_xor((int)sum, 1, 64);
  if ((tid & 1) == 0 && sum) atomicAdd(ws.coarse + (size_t)row * kCoarse + tid / 2, sum);
}

// Bin T of the 128-bin histogram g (scanning from the top) with
// above(T) < need <= above(T) + g[T]; kPassThreads threads call it.
__device__ void pass_find_bin(const uint32_t* __restrict__ g, uint32_t need, uint32_t* s_tot, int* s_bin,
                              uint32_t* s_above) {
  const int tid = threadIdx.x;
  const uint32_t c = tid < kCoarse ? g[kCoarse - 1 - tid] : 0u;
  const uint32_t inc = wave_incl_scan_dpp(c);
  if (lane_id() == 63) s_tot[tid >> 6] = inc;
  if (tid == 0) {   // always overwritten when the counts are consistent
    *s_bin = 0;
    *s_above = 0;
  }
  __syncthreads();
  const uint32_t run = inc - c + (tid >= 64 ? s_tot[0] : 0u);
  if (tid < kCoarse && run < need && run + c >= need) {
    *s_bin = kCoarse - 1 - tid;
    *s_above = run;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kPassThreads) void topk_collect_kernel(const float* __restrict__ scores,
                                                                    const int32_t* __restrict__ row_len,
                                                                    int64_t ld, int k, int vec, PipeWs ws) {
  __shared__ uint32_t s_tot[2][kQuads][kPassWaves];   // per (list, load round, wave) counts
  __shared__ uint32_t s_off[2][kQuads][kPassWaves];
  __shared__ uint32_t s_sum[2];
  __shared__ uint32_t s_w[kPassWaves];
  __shared__ int s_bin;
  __shared__ uint32_t s_above;
  const int row = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int L = (int)min((int64_t)row_len[row], ld);   // row_len <= ld is a precondition
  const int64_t c0 = (int64_t)blockIdx.x * ws.chunk;
  if (L <= k || c0 >= L) return;
  const int t_end = (int)min(c0 + ws.chunk, (int64_t)L);
  const float* s = scores + (size_t)row * ld;
  uint4 kq[kQuads];   // the first round's loads go out before the threshold search
#pragma unroll
  for (int u = 0; u < kQuads; ++u) kq[u] = load_keys4(s, vec != 0, (int)c0 + (u * kPassThreads + tid) * 4, L);
  // threshold bin T of the row: coarse bin, then the fine bin inside it
  pass_find_bin(ws.coarse + (size_t)row * kCoarse, (uint32_t)k, s_w, &s_bin, &s_above);
  const int T0 = s_bin;
  const uint32_t above0 = s_above;
  __syncthreads();
  pass_find_bin(ws.fine + (size_t)row * kFine + T0 * kPerCoarse, (uint32_t)k - above0, s_w, &s_bin, &s_above);
  const uint32_t T = (uint32_t)(T0 * kPerCoarse + s_bin);
  const size_t region = ((size_t)row * ws.chunks + blockIdx.x) * ws.chunk;
  int32_t* sel = ws.sel + region;
  uint2* cand = ws.cand + region;
  uint32_t n_sel = 0, n_cand = 0;   // this chunk's running counts (block-uniform)
  for (int64_t bb = c0; bb < t_end; bb += kBlock) {   // 64-bit: bb + kBlock may pass 2^31 - 1
    const int b = (int)bb;
    if (bb != c0) {
#pragma unroll
      for (int u = 0; u < kQuads; ++u) kq[u] = load_keys4(s, vec != 0, b + (u * kPassThreads + tid) * 4, L);
    }
    // positions ascend with (load round u, wave, lane, element): per-lane
    // flag counts, wave prefix scans, then a prefix over (u, wave)
    uint32_t gt_bits[kQuads], eq_bits[kQuads], ex_gt[kQuads], ex_eq[kQuads];
#pragma unroll
    for (int u = 0; u < kQuads; ++u) {
      const int p = b + (u * kPassThreads + tid) * 4;
      uint32_t g = 0, q = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t d = q_at(kq[u], e) >> kLowBits;
        const bool valid = p + e < t_end;
        g |= (valid && d > T) ? (1u << e) : 0u;
        q |= (valid && d == T) ? (1u << e) : 0u;
      }
      gt_bits[u] = g;
      eq_bits[u] = q;
      const uint32_t cg = (uint32_t)__popc(g), cq = (uint32_t)__popc(q);
      const uint32_t ig = wave_incl_scan_dpp(cg), iq = wave_incl_scan_dpp(cq);
      ex_gt[u] = ig - cg;
      ex_eq[u] = iq - cq;
      if (lane == 63) {
        s_tot[0][u][wave] = ig;
        s_tot[1][u][wave] = iq;
      }
    }
    __syncthreads();
    if (tid < 2) {
      uint32_t v[kQuads * kPassWaves];
#pragma unroll
      for (int i = 0; i < kQuads * kPassWaves; ++i) v[i] = s_tot[tid][i / kPassWaves][i % kPassWaves];
      uint32_t run = 0;
#pragma unroll
      for (int i = 0; i < kQuads * kPassWaves; ++i) {
        s_off[tid][i / kPassWaves][i % kPassWaves] = run;
        run += v[i];
      }
      s_sum[tid] = run;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kQuads; ++u) {
      const int p = b + (u * kPassThreads + tid) * 4;
      uint32_t og = n_sel + s_off[0][u][wave] + ex_gt[u];
      uint32_t oq = n_cand + s_off[1][u][wave] + ex_eq[u];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (gt_bits[u] & (1u << e)) sel[og++] = p + e;
        if (eq_bits[u] & (1u << e)) cand[oq++] = make_uint2(q_at(kq[u], e), (uint32_t)(p + e));
      }
    }
    n_sel += s_sum[0];
    n_cand += s_sum[1];
    __syncthreads();   // s_tot / s_off are rewritten by the next round
  }
  if (tid == 0) ws.counts[(size_t)row * ws.chunks + blockIdx.x] = make_uint2(n_sel, n_cand);
}

struct FinShared {
  uint32_t sel_off[kMaxChunks + 1];
  uint32_t cand_off[kMaxChunks + 1];
  uint32_t hist[1 << kRadix];
  uint32_t wa[kFinWaves], wb[kFinWaves];
  uint32_t misc[4];
};
constexpr size_t kFinListsOff = align_up(sizeof(FinShared), 16);
constexpr size_t kFinLds = kFinListsOff + 2 * (size_t)kMaxK * 4 + (size_t)kCandLds * 8;
static_assert((size_t)kCandLds * 8 >= (size_t)kMaxK * 4, "the candidate area stages the output row");

// Largest c in [0, n) with off[c] <= i, for two lookups at once (off
// ascending, off[0] = 0); fixed steps, both reads issued each step.
__device__ __forceinline__ void chunk_of2(const uint32_t* off_a, uint32_t ia, const uint32_t* off_b, uint32_t ib,
                                          int n, int top, int& ca, int& cb) {
  ca = 0;
  cb = 0;
  for (int step = top; step > 0; step >>= 1) {
    const int ja = ca + step, jb = cb + step;
    const uint32_t va = off_a[min(ja, n - 1)], vb = off_b[min(jb, n - 1)];
    ca = (ja < n && va <= ia) ? ja : ca;
    cb = (jb < n && vb <= ib) ? jb : cb;
  }
}

// Block-wide exclusive prefix of one flag per thread in thread order; returns
// this thread's rank, and the block's total in *total (all threads).
__device__ __forceinline__ uint32_t fin_rank(bool f, uint32_t* wsum, uint32_t* total) {
  const uint64_t m = __ballot(f);
  const int wave = threadIdx.x >> 6;
  if (lane_id() == 0) wsum[wave] = (uint32_t)__popcll(m);
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kFinWaves; ++w) {
    const uint32_t c = wsum[w];
    before += w < wave ? c : 0u;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + mask_rank(m);
}

// Digit T of the 512-bin histogram (scanning from the top) with
// above(T) < need <= above(T) + hist[T]; result in misc[0] (digit) and
// misc[1] (above).
__device__ void fin_find_digit(FinShared& sh, uint32_t need) {
  constexpr int nb = 1 << kRadix;
  constexpr int per = nb > kFinThreads ? nb / kFinThreads : 1;   // bins per thread, descending
  const int tid = threadIdx.x;
  const int hi = nb - 1 - tid * per;
  const bool owns = tid * per < nb;
  uint32_t cnt[per], tot = 0;
#pragma unroll
  for (int j = 0; j < per; ++j) {
    cnt[j] = owns ? sh.hist[hi - j] : 0u;
    tot += cnt[j];
  }
  const uint32_t inc = wave_incl_scan_dpp(tot);
  const int wave = tid >> 6;
  if (lane_id() == 63) sh.wa[wave] = inc;
  if (tid == 0) {   // always overwritten when the counts are consistent
    sh.misc[0] = 0;
    sh.misc[1] = 0;
  }
  __syncthreads();
  uint32_t run = inc - tot;
#pragma unroll
  for (int w = 0; w < kFinWaves; ++w) run += w < wave ? sh.wa[w] : 0u;
#pragma unroll
  for (int j = 0; j < per; ++j) {
    if (owns && run < need && run + cnt[j] >= need) {
      sh.misc[0] = (uint32_t)(hi - j);
      sh.misc[1] = run;
    }
    run += cnt[j];
  }
  __syncthreads();
}

__global__ __launch_bounds__(kFinThreads) void topk_finish_kernel(const int32_t* __restrict__ row_len, int64_t ld,
                                                                  int k, int32_t* __restrict__ idx, PipeWs ws) {
  extern __shared__ __align__(16) unsigned char fin_smem[];
  FinShared& sh = *reinterpret_cast<FinShared*>(fin_smem);
  int32_t* sel = reinterpret_cast<int32_t*>(fin_smem + kFinListsOff);
  int32_t* chosen = sel + kMaxK;
  uint2* cand_l = reinterpret_cast<uint2*>(chosen + kMaxK);
  int32_t* stage = reinterpret_cast<int32_t*>(cand_l);   // output row, once the candidates are used
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int L = (int)min((int64_t)row_len[row], ld);   // row_len <= ld is a precondition
  int32_t* dst = idx + (size_t)row * k;
  if (L <= k) {
    for (int i = tid; i < k; i += kFinThreads) dst[i] = i < L ? i : -1;
    return;
  }
  const int C = (int)(((int64_t)L + ws.chunk - 1) / ws.chunk);
  const uint2* counts = ws.counts + (size_t)row * ws.chunks;
  // exclusive prefix sums of the chunk counts; thread t owns chunks
  // [t*per, t*per + per)
  const int per = (C + kFinThreads - 1) / kFinThreads;   // <= 4
  uint32_t a[4], c[4], ta = 0, tc = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ch = tid * per + j;
    const uint2 n = (j < per && ch < C) ? counts[ch] : make_uint2(0u, 0u);
    a[j] = n.x;
    c[j] = n.y;
    ta += n.x;
    tc += n.y;
  }
  const uint32_t ia = wave_incl_scan_dpp(ta), ic = wave_incl_scan_dpp(tc);
  if (lane_id() == 63) {
    sh.wa[wave] = ia;
    sh.wb[wave] = ic;
  }
  __syncthreads();
  uint32_t ra = ia - ta, rc = ic - tc, A1 = 0, NC = 0;
#pragma unroll
  for (int w = 0; w < kFinWaves; ++w) {
    ra += w < wave ? sh.wa[w] : 0u;
    rc += w < wave ? sh.wb[w] : 0u;
    A1 += sh.wa[w];
    NC += sh.wb[w];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ch = tid * per + j;
    if (j < per && ch < C) {
      sh.sel_off[ch] = ra;
      sh.cand_off[ch] = rc;
    }
    ra += a[j];
    rc += c[j];
  }
  // the counts are exact by construction (A1 < k <= A1 + NC); the clamps
  // only keep broken preconditions (NaN scores) inside the buffers
  A1 = min(A1, (uint32_t)k - 1u);
  const uint32_t need = (uint32_t)k - A1;
  const size_t region0 = (size_t)row * ws.chunks * ws.chunk;
  const int32_t* sel_g = ws.sel + region0;
  const uint2* cand_g = ws.cand + region0;
  constexpr uint32_t kDigitMask = (1u << kRadix) - 1u;
  for (int i = tid; i < (1 << kRadix); i += kFinThreads) sh.hist[i] = 0;
  __syncthreads();
  const bool in_lds = NC <= (uint32_t)kCandLds;
  const int topC = 1 << (31 - __clz(C));   // highest power of two <= C
  auto cand_at_g = [&](uint32_t i) -> uint2 {
    int ch, unused;
    chunk_of2(sh.cand_off, i, sh.cand_off, i, C, topC, ch, unused);
    return cand_g[(size_t)ch * ws.chunk + (i - sh.cand_off[ch])];
  };
  // one pass gathers both lists into LDS (their lookups and loads in flight
  // together) and histograms the candidates' first low digit (bits 17..9)
  const uint32_t n_pass = max(A1, in_lds ? NC : 0u);
  for (uint32_t i = tid; i < n_pass; i += kFinThreads) {
    int cs, cc;
    chunk_of2(sh.sel_off, i, sh.cand_off, i, C, topC, cs, cc);
    const int32_t sv = i < A1 ? sel_g[(size_t)cs * ws.chunk + (i - sh.sel_off[cs])] : 0;
    const uint2 cv = (in_lds && i < NC) ? cand_g[(size_t)cc * ws.chunk + (i - sh.cand_off[cc])] : make_uint2(0u, 0u);
    if (i < A1) sel[i] = sv;
    if (in_lds && i < NC) {
      cand_l[i] = cv;
      atomicAdd(&sh.hist[((cv.x & kLowMask) >> kRadix) & kDigitMask], 1u);
    }
  }
  if (!in_lds)
    for (uint32_t i = tid; i < NC; i += kFinThreads)
      atomicAdd(&sh.hist[((cand_at_g(i).x & kLowMask) >> kRadix) & kDigitMask], 1u);
  __syncthreads();
  auto cand_at = [&](uint32_t i) -> uint2 { return in_lds ? cand_l[i] : cand_at_g(i); };
  // radix select on the low key bits: digit 1 = bits 17..9, digit 2 = 8..0
  fin_find_digit(sh, need);
  uint32_t low_thr = sh.misc[0] << kRadix, above = sh.misc[1];
  __syncthreads();
  for (int i = tid; i < (1 << kRadix); i += kFinThreads) sh.hist[i] = 0;
  __syncthreads();
  for (uint32_t i = tid; i < NC; i += kFinThreads) {
    const uint32_t low = cand_at(i).x & kLowMask;
    if ((low >> kRadix) == (low_thr >> kRadix)) atomicAdd(&sh.hist[low & kDigitMask], 1u);
  }
  __syncthreads();
  fin_find_digit(sh, need - above);
  low_thr |= sh.misc[0];
  above += sh.misc[1];
  __syncthreads();
  // candidates above the threshold are kept, and of those equal to it the
  // first need - above in list (= position) order
  const uint32_t need_eq = need - above;
  uint32_t eq_seen = 0, taken = 0;
  for (uint32_t t0 = 0; t0 < NC && taken < need; t0 += kFinThreads) {
    const uint32_t i = t0 + tid;
    const uint2 x = i < NC ? cand_at(i) : make_uint2(0u, 0u);
    const uint32_t low = x.x & kLowMask;
    const bool gt = i < NC && low > low_thr;
    const bool eq = i < NC && low == low_thr;
    uint32_t n_eq, n_take;
    const uint32_t er = eq_seen + fin_rank(eq, sh.wa, &n_eq);
    const bool take = gt || (eq && er < need_eq);
    const uint32_t slot = taken + fin_rank(take, sh.wb, &n_take);
    if (take && slot < need) chosen[slot] = (int32_t)x.y;
    eq_seen += n_eq;
    taken += n_take;
  }
  __syncthreads();
  // merge: a position's slot is its index in its own list plus the number of
  // entries of the other list below it (the lists are disjoint).  Both
  // searches of a thread run in one fixed-step loop (independent LDS reads).
  const int na = (int)A1, nb = (int)min(taken, need);
  const int nmax = max(na, nb);
  const int top = nmax > 0 ? 1 << (31 - __clz(nmax)) : 0;
  for (int i = tid; i < nmax; i += kFinThreads) {
    const bool va = i < na, vb = i < nb;
    const int32_t xa = va ? sel[i] : 0, xb = vb ? chosen[i] : 0;
    int pa = 0, pb = 0;   // entries of the other list below xa / xb
    for (int step = top; step > 0; step >>= 1) {
      const int ja = pa + step, jb = pb + step;
      const int32_t ca = chosen[max(min(ja, nb) - 1, 0)], cb = sel[max(min(jb, na) - 1, 0)];
      pa = (ja <= nb && ca < xa) ? ja : pa;
      pb = (jb <= na && cb < xb) ? jb : pb;
    }
    if (va) stage[i + pa] = xa;
    if (vb) stage[i + pb] = xb;
  }
  __syncthreads();
  if ((reinterpret_cast<uintptr_t>(dst) & 15u) == 0) {
    const int k4 = k & ~3;
    for (int i = tid * 4; i < k4; i += kFinThreads * 4)
      *reinterpret_cast<uint4*>(dst + i) = *reinterpret_cast<const uint4*>(stage + i);
    for (int i = k4 + tid; i < k; i += kFinThreads) dst[i] = stage[i];
  } else {
    for (int i = tid; i < k; i += kFinThreads) dst[i] = stage[i];
  }
}

// ---------------------------------------------------------------------------
// One-workgroup path for rows whose keys fit in LDS (up to kOneMaxLd
// positions): a single launch.  Longer rows go to the multi-workgroup
// pipeline above, which is faster once the keys no longer fit.  A radix
// select on 12-bit digits (after the bits every key shares) narrows the k-th
// largest key to one bin.  When that bin is small, a bitmap of the kept
// positions is built with ballots and its set bits are emitted in position
// order; otherwise an ordered compaction (each wave owns a contiguous
// position range, ballots give in-order ranks) writes them.  Either way equal
// keys are taken lowest position first and no sort is needed.
// ---------------------------------------------------------------------------
constexpr int kBins = 4096;
constexpr int kOneThreads = 1024;
constexpr int kOneWaves = kOneThreads / 64;
constexpr int kOneLdsKeys = 35840;       // 140 KiB of keys
#ifndef DSA_TOPK_ONE_MAX_LD
#define DSA_TOPK_ONE_MAX_LD kOneLdsKeys
#endif
constexpr int kOneMaxLd = DSA_TOPK_ONE_MAX_LD;   // longest row the one-workgroup path takes
static_assert(kOneMaxLd <= kOneLdsKeys, "the one-workgroup path holds a whole row of keys in LDS");

constexpr int kOneCand = kBins / 4;    // threshold-bin candidates resolved in LDS (first half of hist)
// The candidates are ranked pairwise (one thread each against all), which
// costs O(n^2): past 256 another 12-bit histogram pass is cheaper (a 32K row
// of N(0,1) scores leaves ~500 in its first threshold bin: 40.4 -> 24.2 us
// with the extra pass; indexer scores, whose bins are small, are unchanged).
constexpr int kOneFast = 256;
static_assert(kOneFast <= kOneCand, "the fast path's candidates fit");
constexpr int kOneWords = (kOneLdsKeys + 63) / 64;   // kept-position bitmap (second half of hist)
static_assert(kOneCand * 8 + kOneWords * 8 <= kBins * 4, "candidates and bitmap share the histogram");
static_assert(kOneWords <= kOneThreads, "one bitmap word per thread");

struct OneShared {
  uint32_t hist[kBins];
  uint32_t wave_tot[kOneWaves];
  uint32_t wave_gt[kOneWaves], wave_eq[kOneWaves];
  int bin;
  uint32_t above, count;
  uint32_t ncand, kthr;
  int pthr;
};

// Bin T of an nbins histogram (scanning from the top) with
// above(T) < need <= above(T) + hist[T]; all kOneThreads threads call it.
__device__ void one_find_bin(OneShared& sh, int nbins, uint32_t need) {
  const int tid = threadIdx.x;
  const int per = nbins >= kOneThreads ? nbins / kOneThreads : 1;
  const bool owns = tid * per < nbins;
  const int hi = nbins - 1 - tid * per;
  uint32_t tot = 0;
  if (owns)
    for (int j = 0; j < per; ++j) tot += sh.hist[hi - j];
  const uint32_t inc = wave_incl_scan_dpp(tot);
  const int wave = tid >> 6;
  if (lane_id() == 63) sh.wave_tot[wave] = inc;
  __syncthreads();
  uint32_t run = inc - tot;
#pragma unroll
  for (int w = 0; w < kOneWaves; ++w) run += w < wave ? sh.wave_tot[w] : 0u;   // all reads issued together
  if (owns)
    for (int j = 0; j < per; ++j) {
      const uint32_t c = sh.hist[hi - j];
      if (run < need && run + c >= need) {
        sh.bin = hi - j;
        sh.above = run;
        sh.count = c;
      }
      run += c;
    }
  __syncthreads();
}

__global__ __launch_bounds__(kOneThreads) void topk_one_kernel(const float* __restrict__ scores,
                                                               const int32_t* __restrict__ row_len, int64_t ld,
                                                               int k, int32_t* __restrict__ idx) {
  extern __shared__ __align__(16) unsigned char one_smem[];
  OneShared& sh = *reinterpret_cast<OneShared*>(one_smem);
  uint32_t* keys = reinterpret_cast<uint32_t*>(one_smem + align_up(sizeof(OneShared), 16));
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int L = (int)min((int64_t)row_len[row], ld);   // row_len <= ld is a precondition
  int32_t* dst = idx + (size_t)row * k;
  if (L <= k) {
    for (int i = tid; i < k; i += kOneThreads) dst[i] = i < L ? i : -1;
    return;
  }
  const float* s = scores + (size_t)row * ld;
  constexpr int kU = 8;   // loads in flight per thread
  auto key_at = [&](int t) -> uint32_t { return keys[t]; };
  // Stage the keys (when they fit) and find the key range in the same pass:
  // the bits every key shares are resolved for free, so the first digit
  // spreads over the range the scores actually occupy (indexer scores sit in
  // a few octaves; a fixed top-bits digit would put most of the row into a
  // handful of bins).
  // 16-byte loads (4 positions per lane, a quarter of the load instructions
  // of one position per lane) over the quads inside [0, L); the last L % 4
  // positions, or a row that is not 16-byte aligned, go one by one.
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  const int L4 = (reinterpret_cast<uintptr_t>(s) & 15u) == 0 ? (L & ~3) : 0;
  for (int q0 = tid * 4; q0 < L4; q0 += kU * kOneThreads * 4) {
    float4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = *reinterpret_cast<const float4*>(s + min(q0 + u * kOneThreads * 4, L4 - 4));
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint4 kq = make_uint4(order_key(v[u].x), order_key(v[u].y), order_key(v[u].z), order_key(v[u].w));
      kmin = min(kmin, min(min(kq.x, kq.y), min(kq.z, kq.w)));   // clamped duplicates do not change min/max
      kmax = max(kmax, max(max(kq.x, kq.y), max(kq.z, kq.w)));
      const int q = q0 + u * kOneThreads * 4;
      if (q < L4) *reinterpret_cast<uint4*>(keys + q) = kq;
    }
  }
  for (int t = L4 + tid; t < L; t += kOneThreads) {
    const uint32_t key = order_key(s[t]);
    kmin = min(kmin, key);
    kmax = max(kmax, key);
    keys[t] = key;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
  }
  if (lane == 0) {
    sh.wave_gt[wave] = kmin;
    sh.wave_eq[wave] = kmax;
  }
  __syncthreads();
  kmin = sh.wave_gt[0];
  kmax = sh.wave_eq[0];
  for (int w = 1; w < kOneWaves; ++w) {
    kmin = min(kmin, sh.wave_gt[w]);
    kmax = max(kmax, sh.wave_eq[w]);
  }
  __syncthreads();
  const int common = (kmin ^ kmax) ? __clz(kmin ^ kmax) : 32;
  // radix select: resolved key bits are [31 .. shift]
  int shift = 32 - common;
  uint32_t prefix = shift >= 32 ? 0u : (kmin >> shift) << shift;
  uint32_t need = (uint32_t)k;
  bool fast = false;   // threshold bin small enough to resolve its candidates in LDS
  while (shift > 0) {
    const int nb = min(12, shift);
    const int nshift = shift - nb;
    const uint32_t mask = (1u << nb) - 1u;
    for (int i = tid; i < (1 << nb); i += kOneThreads) sh.hist[i] = 0;
    __syncthreads();
    // four consecutive keys per 16-byte LDS read (the counts do not depend
    // on the order; keys past L up to the next multiple of 4 are read and
    // masked, inside the staging area)
    constexpr int kQ = kU / 4;
    for (int tb = 0; tb < L; tb += kQ * kOneThreads * 4) {
      uint4 kv[kQ];
#pragma unroll
      for (int u = 0; u < kQ; ++u)
        kv[u] = *reinterpret_cast<const uint4*>(keys + min(tb + (u * kOneThreads + tid) * 4, (int)align_up(L, 4) - 4));
#pragma unroll
      for (int u = 0; u < kQ; ++u) {
        const int t = tb + (u * kOneThreads + tid) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = e == 0 ? kv[u].x : e == 1 ? kv[u].y : e == 2 ? kv[u].z : kv[u].w;
          const bool hit = t + e < L && (shift >= 32 || (key >> shift) == (prefix >> shift));
          if (hit) atomicAdd(&sh.hist[(key >> nshift) & mask], 1u);
        }
      }
    }
    __syncthreads();
    one_find_bin(sh, 1 << nb, need);
    need -= sh.above;
    prefix |= (uint32_t)sh.bin << nshift;
    shift = nshift;
    const uint32_t cnt = sh.count;
    __syncthreads();
    if (cnt == need) break;
    if (cnt <= (uint32_t)kOneFast) {
      fast = true;
      break;
    }
  }

  // The kept positions are staged in LDS behind the keys when both fit and
  // then stored 16 bytes per lane (one coalesced pass instead of scattered
  // 4-byte stores); otherwise they are stored directly.
  uint32_t* obuf = keys + align_up(L, 4);
  const bool staged = align_up(L, 4) + align_up(k, 4) <= kOneLdsKeys;
  auto put = [&](uint32_t slot, int t) {
    if (slot >= (uint32_t)k) return;   // exactly k are kept; never write past the row
    if (staged) obuf[slot] = (uint32_t)t;
    else dst[slot] = t;
  };
  auto flush = [&]() {
    if (!staged) return;
    __syncthreads();
    if ((reinterpret_cast<uintptr_t>(dst) & 15u) == 0) {
      const int k4 = k & ~3;
      for (int i = tid * 4; i < k4; i += kOneThreads * 4)
        *reinterpret_cast<uint4*>(dst + i) = *reinterpret_cast<const uint4*>(obuf + i);
      for (int i = k4 + tid; i < k; i += kOneThreads) dst[i] = (int32_t)obuf[i];
    } else {
      for (int i = tid; i < k; i += kOneThreads) dst[i] = (int32_t)obuf[i];
    }
  };

  if (fast) {
    // One pass writes a bitmap of the kept positions: bit t of word t / 64
    // is set where the key's resolved prefix lies above the threshold bin
    // (one ballot per 64 consecutive positions), and the bin's candidates
    // (key, position) are collected.  One thread per candidate ranks it by
    // (key desc, position asc); the first `need` set their bits.  Then
    // thread w emits the set bits of word w in ascending order at the
    // exclusive prefix of the words' popcounts.
    const uint32_t P = prefix >> shift;
    uint2* cand = reinterpret_cast<uint2*>(sh.hist);
    uint64_t* bits = reinterpret_cast<uint64_t*>(sh.hist + 2 * kOneCand);
    const int nwords = (L + 63) / 64;
    if (tid == 0) sh.ncand = 0;
    __syncthreads();
    // wave-uniform loop; the key reads of 8 words are issued together
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    constexpr int kWB = 8;
    for (int w0 = wv; w0 < nwords; w0 += kWB * kOneWaves) {
      uint32_t kk[kWB];
#pragma unroll
      for (int u = 0; u < kWB; ++u) kk[u] = keys[min((w0 + u * kOneWaves) * 64 + lane, L - 1)];
#pragma unroll
      for (int u = 0; u < kWB; ++u) {
        const int wd = w0 + u * kOneWaves;
        if (wd >= nwords) break;
        const int t = wd * 64 + lane;
        const bool valid = t < L;
        const uint32_t kp = kk[u] >> shift;
        const uint64_t gt = __ballot(valid && kp > P);
        const uint64_t eq = __ballot(valid && kp == P);
        if (lane == 0) bits[wd] = gt;
        if (eq) {   // wave-uniform: one slot reservation per wave
          uint32_t base = 0;
          if (lane == 0) base = atomicAdd(&sh.ncand, (uint32_t)__popcll(eq));
          base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
          if (valid && kp == P) {
            const uint32_t slot = base + mask_rank(eq);
            if (slot < (uint32_t)kOneCand) cand[slot] = make_uint2(kk[u], (uint32_t)t);
          }
        }
      }
    }
    __syncthreads();
    const int n = (int)min(sh.ncand, (uint32_t)kOneCand);
    for (int i = tid; i < n; i += kOneThreads) {
      const uint2 c = cand[i];
      uint32_t rank = 0;
      int j = 0;
      for (; j + 8 <= n; j += 8) {   // eight independent reads per step
        uint2 e[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) e[u] = cand[j + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) rank += (e[u].x > c.x || (e[u].x == c.x && e[u].y < c.y)) ? 1u : 0u;
      }
      for (; j < n; ++j) {
        const uint2 e = cand[j];
        rank += (e.x > c.x || (e.x == c.x && e.y < c.y)) ? 1u : 0u;
      }
      if (rank < need) atomicOr(reinterpret_cast<unsigned long long*>(&bits[c.y >> 6]), 1ull << (c.y & 63));
    }
    __syncthreads();
    const uint64_t wb = tid < nwords ? bits[tid] : 0ull;
    const uint32_t c = (uint32_t)__popcll(wb);
    const uint32_t inc = wave_incl_scan_dpp(c);
    if (lane == 63) sh.wave_tot[wave] = inc;
    __syncthreads();
    uint32_t slot = inc - c;
#pragma unroll
    for (int w = 0; w < kOneWaves; ++w) slot += w < wave ? sh.wave_tot[w] : 0u;
    for (uint64_t m = wb; m; m &= m - 1) put(slot++, tid * 64 + __ffsll((long long)m) - 1);
    flush();
    return;
  }

  // ordered compaction: wave w owns positions [w*span, (w+1)*span)
  const int span = ((L + kOneWaves - 1) / kOneWaves + 63) / 64 * 64;
  const int p0 = min(wave * span, L), p1 = min(p0 + span, L);
  const uint32_t P = shift >= 32 ? 0u : (prefix >> shift);
  uint32_t n_gt = 0, n_eq = 0;
  for (int tb = p0; tb < p1; tb += kU * 64) {
    uint32_t kv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) kv[u] = key_at(min(tb + u * 64 + lane, L - 1));
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int t = tb + u * 64 + lane;
      const uint32_t kp = kv[u] >> shift;
      n_gt += __popcll(__ballot(t < p1 && kp > P));
      n_eq += __popcll(__ballot(t < p1 && kp == P));
    }
  }
  if (lane == 0) {
    sh.wave_gt[wave] = n_gt;
    sh.wave_eq[wave] = n_eq;
  }
  __syncthreads();
  uint32_t base_gt = 0, base_eq = 0;
#pragma unroll
  for (int w = 0; w < kOneWaves; ++w) {
    base_gt += w < wave ? sh.wave_gt[w] : 0u;
    base_eq += w < wave ? sh.wave_eq[w] : 0u;
  }
  uint32_t eq_seen = base_eq;
  uint32_t out_pos = base_gt + min(base_eq, need);
  for (int tb = p0; tb < p1; tb += kU * 64) {
    uint32_t kv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) kv[u] = key_at(min(tb + u * 64 + lane, L - 1));
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int t = tb + u * 64 + lane;
      const uint32_t kp = kv[u] >> shift;
      const bool gt = t < p1 && kp > P;
      const bool eq = t < p1 && kp == P;
      const uint64_t eqm = __ballot(eq);
      const bool take = gt || (eq && eq_seen + mask_rank(eqm) < need);
      const uint64_t tm = __ballot(take);
      if (take) put(out_pos + mask_rank(tm), t);
      out_pos += __popcll(tm);
      eq_seen += __popcll(eqm);
    }
  }
  // no padding needed: L > k means exactly k positions were written
  flush();
}

size_t one_lds_bytes() { return align_up(sizeof(OneShared), 16) + (size_t)kOneLdsKeys * 4; }

}  // namespace
}  // namespace dsa

extern "C" size_t dsa_topk_workspace_size(int B, int R, int64_t ld, int k) {
  if (B < 1 || R < 1 || ld < 1 || k < 1) return 0;
  if (ld <= dsa::kOneMaxLd) return 0;
  return dsa::ws_bytes(B * R, ld, nullptr, nullptr);
}

extern "C" dsa_status dsa_topk(const float* scores, const int32_t* row_len, int B, int R, int64_t ld, int k,
                               int32_t* idx, void* workspace, size_t workspace_bytes, void* stream) {
  using namespace dsa;
  clear_error();
  DSA_REQUIRE(scores && row_len && idx, DSA_ERR_INVALID_ARG, "dsa_topk: null pointer argument");
  DSA_REQUIRE(B >= 1 && R >= 1 && ld >= 1 && k >= 1, DSA_ERR_INVALID_ARG,
              "dsa_topk: sizes must be positive (B=%d R=%d ld=%lld k=%d)", B, R, (long long)ld, k);
  DSA_REQUIRE(k <= kMaxK, DSA_ERR_UNSUPPORTED, "dsa_topk: k=%d > %d", k, kMaxK);
  DSA_REQUIRE(ld <= DSA_MAX_LD, DSA_ERR_UNSUPPORTED, "dsa_topk: ld=%lld > %lld", (long long)ld,
              (long long)DSA_MAX_LD);
  DSA_REQUIRE((int64_t)B * R <= 65535, DSA_ERR_UNSUPPORTED, "dsa_topk: B*R=%lld rows > 65535", (long long)B * R);
  const int rows = B * R;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (ld <= kOneMaxLd) {
    // one launch, no workspace
    const size_t lds = one_lds_bytes();
    auto kern = topk_one_kernel;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds) != hipSuccess) {
      set_error("dsa_topk: %zu bytes of LDS not available", lds);
      return DSA_ERR_HIP;
    }
    hipLaunchKernelGGL(kern, dim3(rows), dim3(kOneThreads), lds, s, scores, row_len, ld, k, idx);
    return launch_status("dsa_topk");
  }
  const size_t need = ws_bytes(rows, ld, nullptr, nullptr);
  DSA_REQUIRE(workspace && workspace_bytes >= need, DSA_ERR_WORKSPACE,
              "dsa_topk: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  PipeWs ws;
  ws_bytes(rows, ld, &ws, static_cast<char*>(workspace));
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(topk_finish_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kFinLds) != hipSuccess) {
    set_error("dsa_topk: %zu bytes of LDS not available", kFinLds);
    return DSA_ERR_HIP;
  }
  const int vec = (reinterpret_cast<uintptr_t>(scores) & 15u) == 0 && (ld & 3) == 0;
  const dim3 grid((unsigned)ws.chunks, (unsigned)rows);
  hipLaunchKernelGGL(topk_zero_kernel, dim3(kZeroParts, rows), dim3(kPassThreads), 0, s, ws);
  hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kPassThreads), 0, s, scores, row_len, ld, k, vec, ws);
  hipLaunchKernelGGL(topk_collect_kernel, grid, dim3(kPassThreads), 0, s, scores, row_len, ld, k, vec, ws);
  hipLaunchKernelGGL(topk_finish_kernel, dim3(rows), dim3(kFinThreads), kFinLds, s, row_len, ld, k, idx, ws);
  return launch_status("dsa_topk");
}
