// Top-k selection per (sequence, row) by radix select (gfx950).
//
// DSA glossary entry ("Optimizing speculative decoding", section "IndexShare
// and KVShare"): a top-k selection keeps the most relevant past positions.
// Order: score descending, then position ascending; output ascending, -1 pad.
//
// Scores are mapped to order-preserving 32-bit keys (-0.0 canonicalised to
// +0.0).  The kept set is {key > K*} plus the lowest positions with key == K*,
// where K* is the k-th largest key.  Five launches per call, all multi-
// workgroup except the last:
//   1 zero     clear the per-row histograms and counters
//   2 hist1    histogram of key bits 31..20 (4096 bins; LDS, then integer
//              atomics into the row's global histogram)
//   3 hist2    every workgroup scans hist1 for the threshold bin T1, then
//              histograms key bits 19..8 of the elements in bin T1
//   4 collect  with T1 and T2 known, elements above the 24-bit threshold are
//              appended to the row's `sel` list and those on it to `cand`
//              (wave-aggregated integer atomics; list order is irrelevant)
//   5 finish   one workgroup per row radix-selects the missing elements among
//              the candidates on the composite (key low 8 bits, ~position),
//              merges them with `sel` and bitonic-sorts the kept positions.
// Rows with row_len <= k skip 2-4 and are written directly by 5.
// Integer atomics only: the result is a function of the input set, and the
// final sort makes the output order canonical, so runs are bitwise identical.
#include "dsa_common.h"

namespace dsa {
namespace {

constexpr int kBins = 4096;
constexpr int kHistThreads = 256;
constexpr int kChunk = 4096;          // positions per workgroup in passes 2-4
constexpr int kPerThread = kChunk / kHistThreads;   // 16 loads in flight per thread
constexpr int kFinThreads = 1024;
constexpr int kMaxK = 8192;
constexpr int kCandCap = 8192;        // candidates held in LDS by pass 5

struct RowWs {
  uint32_t* hist1;   // [rows][kBins]
  uint32_t* hist2;   // [rows][kBins]
  uint32_t* cnt;     // [rows][4]: n_sel, n_cand
  int32_t* sel;      // [rows][k]
  uint2* cand;       // [rows][ld]: (key, position)
};

__host__ __device__ inline size_t ws_bytes(int rows, int64_t ld, int k, RowWs* out, char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  size_t h1 = take((size_t)rows * kBins * 4);
  size_t h2 = take((size_t)rows * kBins * 4);
  size_t cn = take((size_t)rows * 4 * 4);
  size_t sl = take((size_t)rows * k * 4);
  size_t cd = take((size_t)rows * ld * 8);
  if (out) {
    out->hist1 = reinterpret_cast<uint32_t*>(base + h1);
    out->hist2 = reinterpret_cast<uint32_t*>(base + h2);
    out->cnt = reinterpret_cast<uint32_t*>(base + cn);
    out->sel = reinterpret_cast<int32_t*>(base + sl);
    out->cand = reinterpret_cast<uint2*>(base + cd);
  }
  return off;
}

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

// Appends `pred` lanes to a list with one atomic per wave; returns the slot
// of this lane (valid where pred).
__device__ __forceinline__ uint32_t wave_append(bool pred, uint32_t* counter) {
  const uint64_t m = __ballot(pred);
  if (m == 0) return 0;
  const int leader = __ffsll((long long)m) - 1;
  uint32_t base = 0;
  if (lane_id() == leader) base = atomicAdd(counter, (uint32_t)__popcll(m));
  base = __shfl(base, leader, 64);
  return base + mask_rank(m);
}

// Threshold bin of a 4096-bin histogram, scanning from the top: the bin T
// with above(T) < need <= above(T) + hist[T].  Run by all kHistThreads
// threads; result in *t_out / *above_out (shared).
__device__ void find_threshold_4096(const uint32_t* hist, uint32_t need, uint32_t* s_wave,
                                    int* t_out, uint32_t* above_out) {
  constexpr int per = kBins / kHistThreads;   // 16 bins per thread
  const int tid = threadIdx.x;
  if (tid == 0) {
    *t_out = 0;
    *above_out = 0;
  }
  // thread tid owns bins [top - per*tid - per + 1, top - per*tid], top = 4095
  const int hi_bin = kBins - 1 - tid * per;
  uint32_t c[per];
  uint32_t tot = 0;
#pragma unroll
  for (int j = 0; j < per; ++j) {
    c[j] = hist[hi_bin - j];
    tot += c[j];
  }
  // inclusive scan over threads (descending bin order)
  const uint32_t inc = wave_incl_scan_dpp(tot);
  const int wave = tid >> 6;
  if (lane_id() == 63) s_wave[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
  for (int wv = 0; wv < wave; ++wv) before += s_wave[wv];
  uint32_t run = before + inc - tot;  // elements in bins above this thread's range
#pragma unroll
  for (int j = 0; j < per; ++j) {
    if (run < need && run + c[j] >= need) {
      *t_out = hi_bin - j;
      *above_out = run;
    }
    run += c[j];
  }
  __syncthreads();
}

__global__ __launch_bounds__(kHistThreads) void topk_zero_kernel(RowWs ws) {
  const int row = blockIdx.x;
  for (int i = threadIdx.x; i < kBins; i += kHistThreads) {
    ws.hist1[(size_t)row * kBins + i] = 0;
    ws.hist2[(size_t)row * kBins + i] = 0;
  }
  if (threadIdx.x < 4) ws.cnt[row * 4 + threadIdx.x] = 0;
}

__global__ __launch_bounds__(kHistThreads) void topk_hist1_kernel(const float* __restrict__ scores,
                                                                  const int32_t* __restrict__ row_len,
                                                                  int64_t ld, int k, RowWs ws) {
  __shared__ uint32_t h[kBins];
  const int row = blockIdx.y;
  const int L = (int)min((int64_t)row_len[row], ld);   // row_len <= ld is a precondition
  const int t0 = blockIdx.x * kChunk;
  if (L <= k || t0 >= L) return;
  for (int i = threadIdx.x; i < kBins; i += kHistThreads) h[i] = 0;
  __syncthreads();
  const float* s = scores + (size_t)row * ld;
  const int t1 = min(t0 + kChunk, L);
  float v[kPerThread];   // all of the chunk's loads in flight at once
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) v[u] = s[min(t0 + (int)threadIdx.x + u * kHistThreads, t1 - 1)];
#pragma unroll
  for (int u = 0; u < kPerThread; ++u)
    if (t0 + (int)threadIdx.x + u * kHistThreads < t1) atomicAdd(&h[order_key(v[u]) >> 20], 1u);
  __syncthreads();
  uint32_t* g = ws.hist1 + (size_t)row * kBins;
  for (int i = threadIdx.x; i < kBins; i += kHistThreads)
    if (h[i]) atomicAdd(&g[i], h[i]);
}

__global__ __launch_bounds__(kHistThreads) void topk_hist2_kernel(const float* __restrict__ scores,
                                                                  const int32_t* __restrict__ row_len,
                                                                  int64_t ld, int k, RowWs ws) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t s_wave[kHistThreads / 64];
  __shared__ int s_t1;
  __shared__ uint32_t s_a1;
  const int row = blockIdx.y;
  const int L = (int)min((int64_t)row_len[row], ld);   // row_len <= ld is a precondition
  const int t0 = blockIdx.x * kChunk;
  if (L <= k || t0 >= L) return;
  for (int i = threadIdx.x; i < kBins; i += kHistThreads) h[i] = 0;
  find_threshold_4096(ws.hist1 + (size_t)row * kBins, (uint32_t)k, s_wave, &s_t1, &s_a1);
  const uint32_t T1 = (uint32_t)s_t1;
  const float* s = scores + (size_t)row * ld;
  const int t1 = min(t0 + kChunk, L);
  float v[kPerThread];
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) v[u] = s[min(t0 + (int)threadIdx.x + u * kHistThreads, t1 - 1)];
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const uint32_t key = order_key(v[u]);
    if (t0 + (int)threadIdx.x + u * kHistThreads < t1 && (key >> 20) == T1) atomicAdd(&h[(key >> 8) & 0xfffu], 1u);
  }
  __syncthreads();
  uint32_t* g = ws.hist2 + (size_t)row * kBins;
  for (int i = threadIdx.x; i < kBins; i += kHistThreads)
    if (h[i]) atomicAdd(&g[i], h[i]);
}

__global__ __launch_bounds__(kHistThreads) void topk_collect_kernel(const float* __restrict__ scores,
                                                                    const int32_t* __restrict__ row_len,
                                                                    int64_t ld, int k, RowWs ws) {
  __shared__ uint32_t s_wave[kHistThreads / 64];
  __shared__ int s_t1, s_t2;
  __shared__ uint32_t s_a1, s_a2;
  __shared__ int32_t l_sel[kChunk];
  __shared__ uint2 l_cand[kChunk];
  __shared__ uint32_t s_n[2], s_base[2];
  const int row = blockIdx.y;
  const int L = (int)min((int64_t)row_len[row], ld);   // row_len <= ld is a precondition
  const int t0 = blockIdx.x * kChunk;
  if (L <= k || t0 >= L) return;
  find_threshold_4096(ws.hist1 + (size_t)row * kBins, (uint32_t)k, s_wave, &s_t1, &s_a1);
  find_threshold_4096(ws.hist2 + (size_t)row * kBins, (uint32_t)k - s_a1, s_wave, &s_t2, &s_a2);
  const uint32_t prefix = ((uint32_t)s_t1 << 12) | (uint32_t)s_t2;  // key bits 31..8
  const float* s = scores + (size_t)row * ld;
  int32_t* sel = ws.sel + (size_t)row * k;
  uint2* cand = ws.cand + (size_t)row * ld;
  uint32_t* cnt = ws.cnt + row * 4;
  const int t1 = min(t0 + kChunk, L);
  // the chunk's selections and candidates are gathered in LDS first; one
  // global atomic per list and workgroup then reserves their place
  if (threadIdx.x < 2) s_n[threadIdx.x] = 0;
  float v[kPerThread];
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) v[u] = s[min(t0 + (int)threadIdx.x + u * kHistThreads, t1 - 1)];
  __syncthreads();
  // whole waves iterate together so the ballots see every lane
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int t = t0 + (int)threadIdx.x + u * kHistThreads;
    const bool valid = t < t1;
    const uint32_t key = order_key(v[u]);
    const uint32_t top = key >> 8;
    const bool is_sel = valid && top > prefix;
    const bool is_cand = valid && top == prefix;
    const uint32_t ps = wave_append(is_sel, &s_n[0]);
    if (is_sel) l_sel[ps] = t;
    const uint32_t pc = wave_append(is_cand, &s_n[1]);
    if (is_cand) l_cand[pc] = make_uint2(key, (uint32_t)t);
  }
  __syncthreads();
  if (threadIdx.x < 2) s_base[threadIdx.x] = s_n[threadIdx.x] ? atomicAdd(&cnt[threadIdx.x], s_n[threadIdx.x]) : 0u;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < s_n[0]; i += kHistThreads)
    if (s_base[0] + i < (uint32_t)k) sel[s_base[0] + i] = l_sel[i];
  for (uint32_t i = threadIdx.x; i < s_n[1]; i += kHistThreads)
    if (s_base[1] + i < (uint32_t)ld) cand[s_base[1] + i] = l_cand[i];
}

// Composite rank of a candidate: key bits 7..0, then ~position (lower
// position ranks higher).  40 bits; bits above are equal for all candidates.
__device__ __forceinline__ uint64_t cand_rank(uint2 c) {
  return ((uint64_t)(c.x & 0xffu) << 32) | (uint64_t)(~c.y);
}

template <bool kInLds>
__device__ void select_candidates(const uint2* cand_g, const uint64_t* cand_l, int n_cand, uint32_t m,
                                  uint32_t* hist, int32_t* out, uint32_t* out_cnt, uint32_t* s_misc) {
  // s_misc[0] = chosen digit, s_misc[1] = count above, s_misc[2] = count equal
  uint64_t prefix = 0;
  int shift = 40;
  uint32_t m_rem = m;
  const int tid = threadIdx.x;
  while (shift > 0) {
    const int nshift = shift - 8;
    for (int i = tid; i < 256; i += kFinThreads) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n_cand; i += kFinThreads) {
      const uint64_t c = kInLds ? cand_l[i] : cand_rank(cand_g[i]);
      if ((c >> shift) == (prefix >> shift)) atomicAdd(&hist[(c >> nshift) & 0xffu], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane owns bins 255-4*lane .. 252-4*lane (descending)
      uint32_t c4[4];
      uint32_t tot = 0;
      for (int j = 0; j < 4; ++j) {
        c4[j] = hist[255 - 4 * tid - j];
        tot += c4[j];
      }
      const uint32_t inc = wave_incl_scan_dpp(tot);
      uint32_t run = inc - tot;
      for (int j = 0; j < 4; ++j) {
        if (run < m_rem && run + c4[j] >= m_rem) {
          s_misc[0] = 255 - 4 * tid - j;
          s_misc[1] = run;
          s_misc[2] = c4[j];
        }
        run += c4[j];
      }
    }
    __syncthreads();
    const uint32_t digit = s_misc[0];
    m_rem -= s_misc[1];
    const uint32_t eq = s_misc[2];
    __syncthreads();
    prefix |= (uint64_t)digit << nshift;
    shift = nshift;
    if (eq == m_rem) break;   // every candidate on this prefix is kept
  }
  for (int i = tid; i < n_cand; i += kFinThreads) {
    const uint64_t c = kInLds ? cand_l[i] : cand_rank(cand_g[i]);
    if ((c >> shift) >= (prefix >> shift)) {
      const uint32_t slot = atomicAdd(out_cnt, 1u);
      if (slot < (uint32_t)kMaxK) out[slot] = (int32_t)(~(uint32_t)c);
    }
  }
  __syncthreads();
}

// Ascending bitonic sort of list[0, 256*E), E elements per thread in
// registers (threads 0..255 hold data; every thread of the block must call
// it, for the barriers).  Strides below E are swaps inside a thread, strides
// below 64*E lane exchanges inside a wave, and only strides of a wave's whole
// span or more go through LDS (two barriers each: 3 of the 66 stages at 2048
// elements, instead of a barrier per stage).
template <int E>
__device__ void sort_regs(int32_t* list) {
  constexpr int P = 256 * E;
  constexpr int WE = 64 * E;
  const int tid = threadIdx.x;
  const bool act = tid < 256;
  const int lane = tid & 63;
  const int base = (tid >> 6) * WE + lane * E;
  int32_t a[E];
  if (act) {
#pragma unroll
    for (int e = 0; e < E; ++e) a[e] = list[base + e];
  }
#pragma unroll
  for (int size = 2; size <= P; size <<= 1) {
#pragma unroll
    for (int stride = size / 2; stride > 0; stride >>= 1) {
      if (stride >= WE) {
        // element i keeps min(a_i, a_{i^stride}) if it is the lower index of
        // an ascending block or the upper index of a descending one, else max
        if (act) {
#pragma unroll
          for (int e = 0; e < E; ++e) list[base + e] = a[e];
        }
        __syncthreads();
        if (act) {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const int i = base + e;
            const int32_t p = list[i ^ stride];
            a[e] = (((i & stride) == 0) == ((i & size) == 0)) ? min(a[e], p) : max(a[e], p);
          }
        }
        __syncthreads();
      } else if (stride >= E) {
        if (act) {
          const int lx = stride / E;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const int i = base + e;
            const int32_t p = __shfl_xor(a[e], lx, 64);
            a[e] = (((i & stride) == 0) == ((i & size) == 0)) ? min(a[e], p) : max(a[e], p);
          }
        }
      } else if (act) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if ((e & stride) == 0) {
            const int32_t x = a[e], y = a[e | stride];
            const bool asc = ((base + e) & size) == 0;
            a[e] = asc ? min(x, y) : max(x, y);
            a[e | stride] = asc ? max(x, y) : min(x, y);
          }
        }
      }
    }
  }
  if (act) {
#pragma unroll
    for (int e = 0; e < E; ++e) list[base + e] = a[e];
  }
  __syncthreads();
}

__global__ __launch_bounds__(kFinThreads) void topk_finish_kernel(const int32_t* __restrict__ row_len, int k,
                                                                  int32_t* __restrict__ idx, RowWs ws,
                                                                  int64_t ld) {
  __shared__ int32_t list[kMaxK];
  __shared__ uint64_t cand_l[kCandCap];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_misc[4];
  __shared__ uint32_t s_cnt;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int L = (int)min((int64_t)row_len[row], ld);   // row_len <= ld is a precondition
  int32_t* dst = idx + (size_t)row * k;
  if (L <= k) {
    for (int i = tid; i < k; i += kFinThreads) dst[i] = i < L ? i : -1;
    return;
  }
  // counts are bounded by construction; the clamps only keep a broken
  // precondition (row_len > ld) from writing out of bounds
  const uint32_t n_sel = min(ws.cnt[row * 4 + 0], (uint32_t)k - 1u);
  const int n_cand = (int)min((int64_t)ws.cnt[row * 4 + 1], ld);
  const uint32_t m = (uint32_t)k - n_sel;
  const int32_t* sel = ws.sel + (size_t)row * k;
  const uint2* cand = ws.cand + (size_t)row * ld;
  for (uint32_t i = tid; i < n_sel; i += kFinThreads) list[i] = sel[i];
  if (tid == 0) s_cnt = n_sel;
  if (n_cand <= kCandCap) {
    for (int i = tid; i < n_cand; i += kFinThreads) cand_l[i] = cand_rank(cand[i]);
    __syncthreads();
    select_candidates<true>(cand, cand_l, n_cand, m, hist, list, &s_cnt, s_misc);
  } else {
    __syncthreads();
    select_candidates<false>(cand, cand_l, n_cand, m, hist, list, &s_cnt, s_misc);
  }
  // bitonic sort of the k kept positions, ascending (in registers when k > 1024)
  int P = 1;
  while (P < k) P <<= 1;
  for (int i = k + tid; i < P; i += kFinThreads) list[i] = 0x7fffffff;
  __syncthreads();
  if (P == 2048) {
    sort_regs<8>(list);
  } else if (P == 4096) {
    sort_regs<16>(list);
  } else if (P == 8192) {
    sort_regs<32>(list);
  } else {
    for (int size = 2; size <= P; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < P / 2; i += kFinThreads) {
          const int lo = 2 * i - (i & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const int32_t a = list[lo], b = list[hi];
          if ((a > b) == up) {
            list[lo] = b;
            list[hi] = a;
          }
        }
        __syncthreads();
      }
    }
  }
  for (int i = tid; i < k; i += kFinThreads) dst[i] = list[i];
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
constexpr int kOneThreads = 1024;
constexpr int kOneWaves = kOneThreads / 64;
constexpr int kOneLdsKeys = 35840;       // 140 KiB of keys
constexpr int kOneMaxLd = kOneLdsKeys;

constexpr int kOneCand = kBins / 4;    // threshold-bin candidates resolved in LDS (first half of hist)
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
    for (int tb = 0; tb < L; tb += kU * kOneThreads) {
      uint32_t kv[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) kv[u] = key_at(min(tb + u * kOneThreads + tid, L - 1));
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int t = tb + u * kOneThreads + tid;
        const uint32_t key = kv[u];
        const bool hit = t < L && (shift >= 32 || (key >> shift) == (prefix >> shift));
        if (hit) atomicAdd(&sh.hist[(key >> nshift) & mask], 1u);
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
    if (cnt <= (uint32_t)kOneCand) {
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
  return dsa::ws_bytes(B * R, ld, k, nullptr, nullptr);
}

extern "C" dsa_status dsa_topk(const float* scores, const int32_t* row_len, int B, int R, int64_t ld, int k,
                               int32_t* idx, void* workspace, size_t workspace_bytes, void* stream) {
  using namespace dsa;
  clear_error();
  DSA_REQUIRE(scores && row_len && idx, DSA_ERR_INVALID_ARG, "dsa_topk: null pointer argument");
  DSA_REQUIRE(B >= 1 && R >= 1 && ld >= 1 && k >= 1, DSA_ERR_INVALID_ARG,
              "dsa_topk: sizes must be positive (B=%d R=%d ld=%lld k=%d)", B, R, (long long)ld, k);
  DSA_REQUIRE(k <= kMaxK, DSA_ERR_UNSUPPORTED, "dsa_topk: k=%d > %d", k, kMaxK);
  DSA_REQUIRE(ld <= ((int64_t)1 << 31) - 1, DSA_ERR_UNSUPPORTED, "dsa_topk: ld too large");
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
  const size_t need = ws_bytes(rows, ld, k, nullptr, nullptr);
  DSA_REQUIRE(workspace && workspace_bytes >= need, DSA_ERR_WORKSPACE,
              "dsa_topk: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  RowWs ws;
  ws_bytes(rows, ld, k, &ws, static_cast<char*>(workspace));
  const unsigned chunks = (unsigned)((ld + kChunk - 1) / kChunk);
  hipLaunchKernelGGL(topk_zero_kernel, dim3(rows), dim3(kHistThreads), 0, s, ws);
  hipLaunchKernelGGL(topk_hist1_kernel, dim3(chunks, rows), dim3(kHistThreads), 0, s, scores, row_len, ld, k, ws);
  hipLaunchKernelGGL(topk_hist2_kernel, dim3(chunks, rows), dim3(kHistThreads), 0, s, scores, row_len, ld, k, ws);
  hipLaunchKernelGGL(topk_collect_kernel, dim3(chunks, rows), dim3(kHistThreads), 0, s, scores, row_len, ld, k, ws);
  hipLaunchKernelGGL(topk_finish_kernel, dim3(rows), dim3(kFinThreads), 0, s, row_len, k, idx, ws, ld);
  return launch_status("dsa_topk");
}
