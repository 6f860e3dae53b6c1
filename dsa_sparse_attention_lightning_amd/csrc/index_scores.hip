// Lightning-indexer scores on bf16 MFMA (gfx950).
//
// DSA glossary entry ("Optimizing speculative decoding", section "IndexShare
// and KVShare"): a light indexer scores every past token with cheap dot
// products.  Scoring form: s_t = sum_h w_h * ReLU(q_h . k_t), one index key
// per position shared by every head.
//
// Mapping.  Per query row the contraction is Q[H x D] * K^T[D x n]: heads are
// the MFMA M dimension, positions the N dimension, the index dimension D the
// K dimension (v_mfma_f32_16x16x32_bf16).  Each wave owns 16, 32 or 64
// positions per step (one to four 16-position N tiles; fewer for small
// problems so that more workgroups run) and streams their keys straight from
// HBM into B fragments: lane l reads 16 contiguous bytes of key row (l % 16) per
// 32-wide K step, so the wave's loads cover whole 256-byte key rows.  The Q
// fragments of every row sit in LDS, already in A-operand lane order, and are
// re-used for every key tile the workgroup streams.  The epilogue (ReLU, * w,
// sum over heads) stays in fp32: a lane holds 4 heads x 1 position per
// 16-head block, sums them, and two cross-lane adds finish the head sum.
#include <type_traits>

#include "dsa_common.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;      // 4 waves

// TILES 16-position MFMA N tiles per wave step; a workgroup step covers
// 4 * 16 * TILES positions.
template <int KS, int MB, int TILES, bool ROWT>
__global__ __launch_bounds__(kThreads) void index_scores_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w,
    const uint16_t* __restrict__ kidx, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ row_len, float* __restrict__ scores, int R, int H,
    int page, int max_pages, int64_t ld, int chunk) {
  constexpr int D = KS * 32;
  constexpr int kWavePos = 16 * TILES;
  constexpr int kBlockPos = kThreads / 64 * kWavePos;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16x8_t* qs = reinterpret_cast<bf16x8_t*>(smem);                 // [R][MB][KS][64]
  float* wl = reinterpret_cast<float*>(smem + (size_t)R * MB * KS * 64 * 16);  // [R][MB*16]

  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  int lmax = 0;
  // row lengths are clamped to what the score rows and the block table can
  // address (a longer row_len is outside the contract; this keeps it in bounds)
  const int cap = (int)min(ld, (int64_t)max_pages * page);
  for (int r = 0; r < R; ++r) lmax = max(lmax, min(row_len[b * R + r], cap));
  const int t_begin = blockIdx.x * chunk;
  if (t_begin >= lmax) return;  // uniform across the workgroup
  const int t_end = min(t_begin + chunk, lmax);
  const int n_iter = (t_end - t_begin + kBlockPos - 1) / kBlockPos;   // >= 1, same for every wave

  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int32_t* bt = block_table + (size_t)b * max_pages;
  // ROWT (several steps per workgroup): the physical key row of every chunk
  // position is resolved once, so later steps' key loads wait on an LDS read
  // instead of a dependent global load
  int* s_row = reinterpret_cast<int*>(wl + R * MB * 16);
  if constexpr (ROWT) {
    for (int i = tid; i < t_end - t_begin; i += kThreads) {
      const int t = t_begin + i;
      s_row[i] = bt[t / page] * page + t % page;
    }
    __syncthreads();
  }

  for (int it = 0; it < n_iter; ++it) {
    const int base = t_begin + it * kBlockPos + wave * kWavePos;
    // key rows straight from HBM into B fragments: lane l holds position
    // base + tile*16 + l%16, dims ks*32 + (l/16)*8 .. +8
    // (positions past t_end load row t_end-1 unconditionally, keeping every
    // load in flight at once; their scores are never stored)
    bf16x8_t bf[TILES][KS];
#pragma unroll
    for (int tile = 0; tile < TILES; ++tile) {
      const int t = min(base + tile * 16 + n, t_end - 1);
      const size_t prow = ROWT ? (size_t)s_row[t - t_begin] : (size_t)bt[t / page] * page + (t % page);
      const uint16_t* src = kidx + prow * D + g * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bf[tile][ks] = *reinterpret_cast<const bf16x8_t*>(src + ks * 32);
    }
    if (it == 0) {
      // Q fragments in A-operand order (issued after the first key loads so
      // the two round trips overlap): fragment (r, mb, ks), lane l holds head
      // mb*16 + l%16, dims ks*32 + (l/16)*8 .. +8.  Heads >= H are zero.
      // Each row's loads read clamped, valid addresses and are masked with
      // bit operations afterwards, so they are all in flight at once (a load
      // under a branch or select of its own is waited for before the next).
      constexpr int kQ = MB * KS * 64;   // fragment slots of one row
      constexpr int kQPer = (kQ + kThreads - 1) / kThreads;
      constexpr int kW = MB * 16;
      for (int r = 0; r < R; ++r) {
        uint4 v[kQPer];
        uint32_t keep[kQPer];
#pragma unroll
        for (int j = 0; j < kQPer; ++j) {
          const int i = min(tid + j * kThreads, kQ - 1);
          const int fl = i & 63;
          const int f = i >> 6;
          const int ks = f % KS;
          const int mb = f / KS;
          const int h = mb * 16 + (fl & 15);
          keep[j] = h < H ? ~0u : 0u;
          v[j] = *reinterpret_cast<const uint4*>(q + ((size_t)(b * R + r) * H + min(h, H - 1)) * D + ks * 32 +
                                                 (fl >> 4) * 8);
        }
        const int wh = tid % kW;
        const float wv = w[(size_t)(b * R + r) * H + min(wh, H - 1)];
        __builtin_amdgcn_sched_barrier(0);   // every load above is issued before any is used
#pragma unroll
        for (int j = 0; j < kQPer; ++j) {
          const int i = tid + j * kThreads;
          if (kQ % kThreads == 0 || i < kQ) {
            const uint4 m = make_uint4(v[j].x & keep[j], v[j].y & keep[j], v[j].z & keep[j], v[j].w & keep[j]);
            reinterpret_cast<uint4*>(qs)[r * kQ + i] = m;
          }
        }
        // threads tid, tid + kW, ... store the same weight into the same slot
        wl[r * kW + wh] = __uint_as_float(__float_as_uint(wv) & (wh < H ? ~0u : 0u));
      }
      __syncthreads();
    }
    for (int r = 0; r < R; ++r) {
      float sacc[TILES];
#pragma unroll
      for (int tile = 0; tile < TILES; ++tile) sacc[tile] = 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        f32x4_t acc[TILES];
#pragma unroll
        for (int tile = 0; tile < TILES; ++tile) acc[tile] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8_t a = qs[((r * MB + mb) * KS + ks) * 64 + lane];
#pragma unroll
          for (int tile = 0; tile < TILES; ++tile)
            acc[tile] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bf[tile][ks], acc[tile], 0, 0, 0);
        }
        // lane holds heads mb*16 + g*4 + {0..3} for position n of each tile
        const float4 wv = *reinterpret_cast<const float4*>(&wl[r * MB * 16 + mb * 16 + g * 4]);
#pragma unroll
        for (int tile = 0; tile < TILES; ++tile) {
          float sum = sacc[tile];
          sum += wv.x * fmaxf(acc[tile][0], 0.f);
          sum += wv.y * fmaxf(acc[tile][1], 0.f);
          sum += wv.z * fmaxf(acc[tile][2], 0.f);
          sum += wv.w * fmaxf(acc[tile][3], 0.f);
          sacc[tile] = sum;
        }
      }
      // finish the head sum across the four lane groups
#pragma unroll
      for (int tile = 0; tile < TILES; ++tile) {
        float sum = sacc[tile];
        sum += __shfl_xor(sum, 16, 64);
        sum += __shfl_xor(sum, 32, 64);
        sacc[tile] = sum;
      }
      // lane group g writes tile g (positions base + g*16 + n)
      float mine = sacc[0];
#pragma unroll
      for (int tile = 1; tile < TILES; ++tile)
        if (g == tile) mine = sacc[tile];
      const int t = base + g * 16 + n;
      if (g < TILES && t < t_end && t < row_len[b * R + r]) scores[(size_t)(b * R + r) * ld + t] = mine;   // t_end <= cap
    }
  }
}

template <int KS, int MB, int TILES>
dsa_status launch_index_t(const void* q, const float* w, const void* kidx, const int32_t* bt,
                          const int32_t* row_len, float* scores, int B, int R, int H, int page,
                          int max_pages, int64_t ld, hipStream_t stream) {
  constexpr int kBlockPos = kThreads / 64 * 16 * TILES;
  // Positions per workgroup: whole steps, sized so that a long row still
  // spreads over about 4096 workgroups (2048: 0.5-2 us slower at 2^20 and on
  // the 16-sequence batch).
#ifndef DSA_INDEX_TARGET_WGS
#define DSA_INDEX_TARGET_WGS 4096
#endif
  const int64_t steps = (ld + kBlockPos - 1) / kBlockPos;
  int per = (int)((steps * B + DSA_INDEX_TARGET_WGS - 1) / DSA_INDEX_TARGET_WGS);
  per = per < 1 ? 1 : per > 8 ? 8 : per;
  const bool rowt = per > 1;
  const size_t lds = (size_t)R * MB * KS * 64 * 16 + (size_t)R * MB * 16 * sizeof(float) +
                     (rowt ? (size_t)per * kBlockPos * sizeof(int) : 0);
  auto kern = rowt ? index_scores_kernel<KS, MB, TILES, true> : index_scores_kernel<KS, MB, TILES, false>;
  if (lds > 65536) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
      set_error("dsa_index_scores: %zu bytes of LDS not available", lds);
      return DSA_ERR_UNSUPPORTED;
    }
  }
  const int chunk = per * kBlockPos;
  const int64_t gx = (ld + chunk - 1) / chunk;
  dim3 grid((unsigned)gx, (unsigned)B);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, stream,
                     static_cast<const uint16_t*>(q), w, static_cast<const uint16_t*>(kidx), bt,
                     row_len, scores, R, H, page, max_pages, ld, chunk);
  return launch_status("dsa_index_scores");
}

template <int KS, int MB>
dsa_status launch_index(const void* q, const float* w, const void* kidx, const int32_t* bt,
                        const int32_t* row_len, float* scores, int B, int R, int H, int page,
                        int max_pages, int64_t ld, hipStream_t stream) {
  // small problems: one 16-position tile per wave step, so more workgroups;
  // otherwise two (eight key loads in flight per lane; four tiles per step
  // measured 2-4 us slower at 2^20 and on the 16-sequence batch)
  const int64_t total = ld * (int64_t)B;
  if (total <= (1 << 18))
    return launch_index_t<KS, MB, 1>(q, w, kidx, bt, row_len, scores, B, R, H, page, max_pages, ld, stream);
  return launch_index_t<KS, MB, 2>(q, w, kidx, bt, row_len, scores, B, R, H, page, max_pages, ld, stream);
}

// ---------------------------------------------------------------------------
// Several query rows (R >= 2, e.g. the verify-pass shape with one row per
// chained position): the contraction has M = R * 64 (row, head) pairs, so it
// is a real GEMM.  Wave w owns query row w = 2 M blocks of 32 (row, head)
// pairs, whose Q fragments stay in registers for the whole kernel.  The
// workgroup stages 32-position key tiles in LDS once for all its waves (the
// next tile is prefetched into registers while the current one is consumed)
// and every wave runs v_mfma_f32_32x32x16_bf16 over them.  Epilogue as in the
// one-row kernel: ReLU, * w, head sum in fp32 (16 heads per lane, then the
// two lane halves).
// C layout of the 32x32 MFMA: lane l, register v holds row (v/4)*8 +
// (l/32)*4 + v%4, column l%32.
// ---------------------------------------------------------------------------
constexpr int kRowsTile = 32;
constexpr int kMaxChunkPositions = 4096;   // per-workgroup chunk cap (LDS row table)

#ifndef DSA_INDEX_WPE
#define DSA_INDEX_WPE 2
#endif
template <int KS16, int NWAVE>
__global__ __launch_bounds__(NWAVE * 64) __attribute__((amdgpu_waves_per_eu(DSA_INDEX_WPE))) void index_scores_rows_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ kidx,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ row_len, float* __restrict__ scores,
    int R, int H, int page, int max_pages, int64_t ld, int chunk) {
  constexpr int D = KS16 * 16;
  constexpr int NT = NWAVE * 64;
  constexpr int MBW = 2;                             // 32-row M blocks per wave (one row)
  constexpr int KROW = D * 2 + 16;                   // padded LDS row (bytes)
  constexpr int CHUNKS = kRowsTile * D / 8;          // 16-byte pieces per tile
  constexpr int PER = (CHUNKS + NT - 1) / NT;
  __shared__ __align__(16) unsigned char s_k[2 * kRowsTile * KROW];
  __shared__ __align__(16) float s_w[NWAVE][64];
  __shared__ int s_row[kMaxChunkPositions];   // physical key row of each chunk position

  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  int lmax = 0;
  // row lengths are clamped to what the score rows and the block table can
  // address (a longer row_len is outside the contract; this keeps it in bounds)
  const int cap = (int)min(ld, (int64_t)max_pages * page);
  for (int r = 0; r < R; ++r) lmax = max(lmax, min(row_len[b * R + r], cap));
  const int t_begin = blockIdx.x * chunk;
  if (t_begin >= lmax) return;
  const int t_end = min(t_begin + chunk, lmax);
  const int32_t* bt = block_table + (size_t)b * max_pages;
  // physical row of every chunk position, resolved once through the block
  // table (a key load then needs no dependent global load and no division)
  for (int i = tid; i < t_end - t_begin; i += NT) {
    const int t = t_begin + i;
    s_row[i] = bt[t / page] * page + t % page;
  }
  // how far this lane's row is valid (read before the tile loop, so that the
  // loop's only global loads are the key prefetches); the low lane half stores
  const int t_lim = (wave < R && hi == 0) ? min(t_end, row_len[b * R + wave]) : 0;

  // Q fragments: block mb = row w, heads mb*32 + l%32
  bf16x8_t qa[MBW][KS16];
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb) {
    const int r = wave;
    const int h = mb * 32 + l32;
    const bool ok = r < R && h < H;
    const uint16_t* src = q + ((size_t)(b * R + (ok ? r : 0)) * H + (ok ? h : 0)) * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS16; ++ks)
      qa[mb][ks] = ok ? *reinterpret_cast<const bf16x8_t*>(src + ks * 16) : bf16x8_t{};
  }
  for (int i = tid; i < NWAVE * 64; i += NT) {
    const int r = i / 64, h = i % 64;
    s_w[r][h] = (r < R && h < H) ? 0.5f * w[(size_t)(b * R + r) * H + h] : 0.f;
  }

  // key tile loads: piece c = tid + j*NT -> position c / (D/8), 16-byte
  // column c % (D/8).  A ring of PF tiles is in flight in registers; the LDS
  // tile is double-buffered so one barrier per tile suffices.
  constexpr int PF = 4;
  struct Slot {
    uint4 v[PER];
  };
  auto fetch = [&](int t0) __attribute__((always_inline)) {
    Slot out;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int c = min(tid + j * NT, CHUNKS - 1);
      const int t = min(t0 + c / (D / 8), t_end - 1);
      const uint16_t* src = kidx + (size_t)s_row[t - t_begin] * D + (c % (D / 8)) * 8;
      out.v[j] = *reinterpret_cast<const uint4*>(src);
    }
    return out;
  };
  const int n_tiles = (t_end - t_begin + kRowsTile - 1) / kRowsTile;
  // one tile: stage it from its ring slot, refill the slot PF tiles ahead,
  // run the MFMAs and the epilogue
  auto tile_step = [&](Slot slot, int tile_no) __attribute__((always_inline)) {
    const int t0 = t_begin + tile_no * kRowsTile;
    unsigned char* buf = s_k + (tile_no & 1) * (kRowsTile * KROW);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int c = tid + j * NT;
      if (CHUNKS % NT == 0 || c < CHUNKS) *reinterpret_cast<uint4*>(buf + (c / (D / 8)) * KROW + (c % (D / 8)) * 16) = slot.v[j];
    }
    __syncthreads();
    const Slot next = fetch(t0 + PF * kRowsTile);   // clamped inside the chunk; tiles past t_end are never stored

    f32x16_t acc[MBW];
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) acc[mb] = f32x16_t{};
    // B fragment of the next k step read while the current one multiplies
    const unsigned char* brow = buf + l32 * KROW + hi * 16;
    bf16x8_t kb = *reinterpret_cast<const bf16x8_t*>(brow);
#pragma unroll
    for (int ks = 0; ks < KS16; ++ks) {
      bf16x8_t kn = kb;
      if (ks + 1 < KS16) kn = *reinterpret_cast<const bf16x8_t*>(brow + (ks + 1) * 32);
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][ks], kb, acc[mb], 0, 0, 0);
      kb = kn;
    }
    // epilogue: rows of block mb are heads (mb%2)*32 + (v/4)*8 + hi*4 + v%4
    float part = 0.f;
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // s_w holds w/2, and (x + |x|) * (w/2) equals w * ReLU(x) exactly
        // (power-of-two scaling), without a compare per element
        const float4 wv = *reinterpret_cast<const float4*>(&s_w[wave][mb * 32 + g * 8 + hi * 4]);
        part = fmaf(wv.x, acc[mb][g * 4 + 0] + fabsf(acc[mb][g * 4 + 0]), part);
        part = fmaf(wv.y, acc[mb][g * 4 + 1] + fabsf(acc[mb][g * 4 + 1]), part);
        part = fmaf(wv.z, acc[mb][g * 4 + 2] + fabsf(acc[mb][g * 4 + 2]), part);
        part = fmaf(wv.w, acc[mb][g * 4 + 3] + fabsf(acc[mb][g * 4 + 3]), part);
      }
    }
    part += __shfl_xor(part, 32, 64);
    // the low lane half stores row `wave`
    const int t = t0 + l32;
    const float v = part;
    if (t < t_lim) scores[(size_t)(b * R + wave) * ld + t] = v;
    return next;
  };
  __syncthreads();   // s_row, s_w ready
  Slot pre0 = fetch(t_begin);
  Slot pre1 = fetch(t_begin + kRowsTile);
  Slot pre2 = fetch(t_begin + 2 * kRowsTile);
  Slot pre3 = fetch(t_begin + 3 * kRowsTile);
  // whole rounds of PF tiles, then the tail (keeping the loop body free of
  // branches lets every wait cover only the slot that is consumed)
  int tg = 0;
  for (; tg + PF <= n_tiles; tg += PF) {
    pre0 = tile_step(pre0, tg);
    pre1 = tile_step(pre1, tg + 1);
    pre2 = tile_step(pre2, tg + 2);
    pre3 = tile_step(pre3, tg + 3);
  }
  if (tg < n_tiles) tile_step(pre0, tg);   // n_tiles - tg is uniform across the workgroup
  if (tg + 1 < n_tiles) tile_step(pre1, tg + 1);
  if (tg + 2 < n_tiles) tile_step(pre2, tg + 2);
}

// Five to eight rows: eight waves, one query row each (Q fragments 64 VGPRs,
// head weights 16, two accumulator sets 64), two waves per SIMD.  Key tiles
// are staged in LDS four at a time (128 positions per barrier; the next
// stage's loads are in flight in registers while the current one is used:
// one stage ahead measured 2 % faster than two, with 24 fewer VGPRs), and
// each wave software-pipelines its tiles: the
// MFMAs of tile i issue while its VALU runs the epilogue of tile i-1 out of
// the other accumulator set, with the weights in registers (no LDS access in
// the epilogue).  The contraction runs on v_mfma_f32_16x16x32_bf16 (four
// 16-head blocks x two 16-position blocks per 32-position tile): on
// full-mantissa operands, where the chip clocks down under MFMA load, it
// sustains 10-20 % more than the 32x32x16 form (register-only loops), and
// this kernel runs about 1-2 % faster with it.  Same ReLU * w epilogue as
// index_scores_rows_kernel; the head sum is taken in a different order.
#ifndef DSA_INDEX_SUPER_WGS
#define DSA_INDEX_SUPER_WGS 256
#endif
#ifndef DSA_INDEX_SUPER_TILES
#define DSA_INDEX_SUPER_TILES 4
#endif
constexpr int kSuperTiles = DSA_INDEX_SUPER_TILES;    // 32-position tiles per LDS stage (even)
constexpr int kSuperPos = kSuperTiles * kRowsTile;    // positions per stage
#ifndef DSA_INDEX_SUPER_PF
#define DSA_INDEX_SUPER_PF 1
#endif
constexpr int kSuperPF = DSA_INDEX_SUPER_PF;          // stages in flight in registers (1 or 2)
constexpr int kSuperThreads = 512;

template <int KS16>
constexpr size_t super_lds_bytes() {
  return (size_t)2 * kSuperPos * (KS16 * 32 + 16);
}

template <int KS16>
__global__ __launch_bounds__(kSuperThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void index_scores_rows8_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ kidx,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ row_len, float* __restrict__ scores,
    int R, int H, int page, int max_pages, int64_t ld, int chunk) {
  constexpr int NT = kSuperThreads;
  constexpr int MB = 4;                                // 16-head M blocks of the wave's row
  constexpr int NB = kRowsTile / 16;                   // 16-position N blocks of a tile
  constexpr int D = KS16 * 16;
  constexpr int KS = D / 32;                           // 32-wide K steps
  static_assert(KS >= 1, "D_I is a multiple of 32");
  constexpr int KROW = D * 2 + 16;                     // padded LDS row (bytes)
  constexpr int CHUNKS = kSuperPos * D / 8;            // 16-byte pieces per stage
  static_assert(CHUNKS % NT == 0, "stage pieces must divide evenly");
  static_assert(kSuperTiles == 2 || kSuperTiles == 4 || kSuperTiles == 8, "2, 4 or 8 tiles per stage");
  static_assert(kMaxChunkPositions % kSuperPos == 0, "chunks are whole stages");
  constexpr int PER = CHUNKS / NT;
  constexpr int EPS = 32 / (KS * NB * MB);             // epilogue elements per MFMA slot
  constexpr int PF = kSuperPF;                         // stages in flight
  extern __shared__ __align__(16) unsigned char s_k[];   // [2][kSuperPos][KROW]
  // byte offset of each chunk position's key row; the slots past the chunk
  // (the PF + 1 stages read ahead and never used, and the rounding to whole
  // fill rounds) hold the chunk's first row
  constexpr int kTable = (kMaxChunkPositions + (PF + 1) * kSuperPos + NT - 1) / NT * NT;
  __shared__ int64_t s_off[kTable];

  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;   // 16x16x32 layout: A row / B column / C column
  const int g4 = lane >> 4;    // K group (A, B) and C row group
  // Start-up: every load of the prologue (Q fragments, weights, row lengths,
  // the block-table entries of this thread's table slots and of its stage-0
  // key pieces) reads a clamped, valid address and is issued before any of
  // them is used; the scheduling fence keeps the compiler from pairing each
  // load with its use, which would wait for the loads one at a time.
  // Block-table entries are read before the chunk bounds are known; slots
  // past the chunk's end are replaced below by the chunk's first row.
  const int wrow = b * R + min(wave, R - 1);
  const int cap = (int)min(ld, (int64_t)max_pages * page);
  const int t_begin = blockIdx.x * chunk;
  const int32_t* bt = block_table + (size_t)b * max_pages;
  constexpr int kFill = kTable / NT;
  auto pos_c = [&](int t) __attribute__((always_inline)) { return min(t, cap - 1); };
  // Rows past R read a valid row's query (never stored); heads past H read a
  // valid head's query, zeroed after the fence, with weight 0.
  // A fragment (mb, ks): lane l holds head mb*16 + l%16, dims ks*32 +
  // (l/16)*8 .. +8.  C register i of block mb holds head mb*16 + (l/16)*4 + i.
  bf16x8_t qa[MB][KS];
  float wraw[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int h = mb * 16 + l16;
    const uint16_t* src = q + ((size_t)wrow * H + min(h, H - 1)) * D + g4 * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[mb][ks] = *reinterpret_cast<const bf16x8_t*>(src + ks * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) wraw[mb][i] = w[(size_t)wrow * H + min(mb * 16 + g4 * 4 + i, H - 1)];
  }
  const int my_len = row_len[wrow];
  int rl[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) rl[r] = row_len[b * R + min(r, R - 1)];
  int pbt[kFill];   // this thread's table slots
#pragma unroll
  for (int k = 0; k < kFill; ++k) pbt[k] = bt[pos_c(t_begin + tid + k * NT) / page];
  int sbt[PER];     // this thread's stage-0 key pieces
#pragma unroll
  for (int j = 0; j < PER; ++j) sbt[j] = bt[pos_c(t_begin + (tid + j * NT) / (D / 8)) / page];
  const int fbt = bt[pos_c(t_begin) / page];
  __builtin_amdgcn_sched_barrier(0);

  float wr[MB][4];   // w/2 of the heads this lane's accumulator registers hold
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hv = mb * 16 + g4 * 4 + i;
      wr[mb][i] = (wave < R && hv < H) ? 0.5f * wraw[mb][i] : 0.f;
    }
    const uint32_t keep = mb * 16 + l16 < H ? ~0u : 0u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 v = __builtin_bit_cast(uint4, qa[mb][ks]);
      qa[mb][ks] = __builtin_bit_cast(bf16x8_t, make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep));
    }
  }
  auto row_at = [&](int e, int t) __attribute__((always_inline)) {
    return (int)((uint32_t)e * (uint32_t)page + (uint32_t)(pos_c(t) % page));
  };
  const int first_row = row_at(fbt, t_begin);
  int64_t poff[kFill];   // byte offsets of the table slots' rows, selected below
#pragma unroll
  for (int k = 0; k < kFill; ++k) poff[k] = (int64_t)row_at(pbt[k], t_begin + tid + k * NT) * (D * 2);
  int64_t soff[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) soff[j] = (int64_t)row_at(sbt[j], t_begin + (tid + j * NT) / (D / 8)) * (D * 2);
  int lmax = 0;
#pragma unroll
  for (int r = 0; r < 8; ++r) lmax = max(lmax, min(rl[r], cap));
  // No early exit here: a branch on the row lengths is hoisted by the
  // compiler above the other loads and would serialize two round trips.  A
  // chunk past every row (only when ld exceeds all row lengths) instead runs
  // one stage on keys read from the start of q (valid memory; its block-table
  // entries may not be) and stores nothing.
  const bool empty = t_begin >= lmax;
  const int t_end = empty ? t_begin : min(t_begin + chunk, lmax);
  const int len = t_end - t_begin;
  const int64_t first_off = empty ? 0 : (int64_t)first_row * (D * 2);
#pragma unroll
  for (int k = 0; k < kFill; ++k) {
    const int i = tid + k * NT;
    s_off[i] = i < len ? poff[k] : first_off;
  }
  // wave w owns row w; after the head sum, lane groups 0 and 2 store the
  // tile's two 16-position blocks
  const int tpos = (g4 >> 1) * 16 + l16;
  const int t_lim = (!empty && wave < R && (g4 & 1) == 0) ? min(t_end, my_len) : 0;

  struct Slot {
    uint4 v[PER];
  };
  // key-row byte offsets of the stage fetched next, read one stage ahead of
  // use; a thread's 16-byte piece of a row is the same in every load
  static_assert(NT % (D / 8) == 0, "each thread keeps one piece of the key rows");
  const unsigned char* kbase =
      reinterpret_cast<const unsigned char*>(empty ? static_cast<const void*>(q) : static_cast<const void*>(kidx)) +
      (tid % (D / 8)) * 16;
  int64_t koff[PER];
  auto read_rows = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < PER; ++j) koff[j] = s_off[st * kSuperPos + (tid + j * NT) / (D / 8)];
  };
  auto fetch = [&]() __attribute__((always_inline)) {
    Slot out;
#pragma unroll
    for (int j = 0; j < PER; ++j) out.v[j] = *reinterpret_cast<const uint4*>(kbase + koff[j]);
    return out;
  };
  // stage 0's key pieces are fetched from the block-table entries directly,
  // without waiting for the table
#pragma unroll
  for (int j = 0; j < PER; ++j)
    koff[j] = (tid + j * NT) / (D / 8) < len ? soff[j] : first_off;
  Slot pre0 = fetch();
  __syncthreads();   // s_off ready
  const f32x4_t zero{};
  // p0, p1: this lane's partial head sums (16 heads) of positions l%16 of
  // the tile's two blocks; the four lane groups hold disjoint heads
  auto epilogue_store = [&](float p0, float p1, int g) __attribute__((always_inline)) {
    // lanes 0-31 add groups (0,2) and (1,3) of block 0, lanes 32-63 those of
    // block 1; then lane l adds lane l ^ 16: all four groups.  Both
    // exchanges are VALU lane swaps (a shuffle through the LDS crossbar
    // would wait for the fragment reads in flight).
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
    const float v1 = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const auto sw16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v1), __float_as_uint(v1), false, false);
    const float v = __uint_as_float(sw16[0]) + __uint_as_float(sw16[1]);
    const int t = t_begin + g * kRowsTile + tpos;
    // scores are not re-read here: non-temporal stores (measured 4-5 % faster
    // than stores that allocate in the last-level cache)
    if (t < t_lim) __builtin_nontemporal_store(v, &scores[(size_t)(b * R + wave) * ld + t]);
  };
  // element e of a tile's accumulators: block nb = e/16, head block
  // mb = (e/4)%4, register e%4
  auto epi_elem = [&](const f32x4_t (&accP)[NB * MB], int e, float& p0, float& p1) __attribute__((always_inline)) {
    const int nb = e / 16, mb = (e / 4) % MB, i = e % 4;
    const float x = accP[nb * MB + mb][i];
    // (x + |x|) * (w/2) equals w * ReLU(x) exactly
    if (nb == 0) p0 = fmaf(wr[mb][i], x + fabsf(x), p0);
    else p1 = fmaf(wr[mb][i], x + fabsf(x), p1);
  };
  // B fragments of a stage are read in order f = (u * KS + ks) * NB + nb
  // (tile u, k step ks, block nb) through a ring, BPF fragments ahead of
  // their MFMAs; fragment (nb, ks): lane l holds position nb*16 + l%16,
  // dims ks*32 + (l/16)*8 .. +8
  constexpr int BPF = 2;
  constexpr int NF = kSuperTiles * KS * NB;
  bf16x8_t kf[BPF + 1];
  auto frag = [&](const unsigned char* bbase, int f) __attribute__((always_inline)) {
    const int u = f / (KS * NB), ks = (f / NB) % KS, nb = f % NB;
    return *reinterpret_cast<const bf16x8_t*>(bbase + (u * kRowsTile + nb * 16) * KROW + ks * 64);
  };
  // tile U of the stage (global tile g): MFMAs into accC and, interleaved
  // with them, the epilogue of tile g-1 out of accP
  auto tile = [&](auto has_prev, auto u_c, const unsigned char* bbase, int g, f32x4_t (&accC)[NB * MB],
                  f32x4_t (&accP)[NB * MB]) __attribute__((always_inline)) {
    constexpr bool EPI = decltype(has_prev)::value;
    constexpr int U = decltype(u_c)::value;
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int f = (U * KS + ks) * NB + nb;
        if (f + BPF < NF) kf[(f + BPF) % (BPF + 1)] = frag(bbase, f + BPF);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          accC[nb * MB + mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mb][ks], kf[f % (BPF + 1)],
                                                                        ks == 0 ? zero : accC[nb * MB + mb], 0, 0, 0);
          if constexpr (EPI) {
#pragma unroll
            for (int e = 0; e < EPS; ++e) epi_elem(accP, ((ks * NB + nb) * MB + mb) * EPS + e, p0, p1);
          }
        }
      }
    }
    if constexpr (EPI) epilogue_store(p0, p1, g - 1);
  };
  using no_prev = std::integral_constant<bool, false>;
  using with_prev = std::integral_constant<bool, true>;
  f32x4_t accA[NB * MB], accB[NB * MB];
  // one stage: store it to LDS, prefetch PF stages ahead, run its four tiles
  // (even tiles in set A, odd in set B)
  auto step = [&](auto first, Slot slot, int st) __attribute__((always_inline)) {
    unsigned char* buf = s_k + (st & 1) * (kSuperPos * KROW);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int c = tid + j * NT;
      *reinterpret_cast<uint4*>(buf + (c / (D / 8)) * KROW + (c % (D / 8)) * 16) = slot.v[j];
    }
    __syncthreads();
    const Slot next = fetch();   // stage st + PF (rows read last step)
    read_rows(st + PF + 1);
    const unsigned char* bbase = buf + l16 * KROW + g4 * 16;
#pragma unroll
    for (int f = 0; f < BPF; ++f) kf[f] = frag(bbase, f);
    const int g = st * kSuperTiles;
    if constexpr (decltype(first)::value) tile(no_prev{}, std::integral_constant<int, 0>{}, bbase, g, accA, accB);
    else tile(with_prev{}, std::integral_constant<int, 0>{}, bbase, g, accA, accB);
    tile(with_prev{}, std::integral_constant<int, 1>{}, bbase, g + 1, accB, accA);
    if constexpr (kSuperTiles >= 4) {
      tile(with_prev{}, std::integral_constant<int, 2>{}, bbase, g + 2, accA, accB);
      tile(with_prev{}, std::integral_constant<int, 3>{}, bbase, g + 3, accB, accA);
    }
    if constexpr (kSuperTiles >= 8) {
      tile(with_prev{}, std::integral_constant<int, 4>{}, bbase, g + 4, accA, accB);
      tile(with_prev{}, std::integral_constant<int, 5>{}, bbase, g + 5, accB, accA);
      tile(with_prev{}, std::integral_constant<int, 6>{}, bbase, g + 6, accA, accB);
      tile(with_prev{}, std::integral_constant<int, 7>{}, bbase, g + 7, accB, accA);
    }
    return next;
  };
  using first_stage = std::integral_constant<bool, true>;
  using later_stage = std::integral_constant<bool, false>;
  const int n_st = max(1, (len + kSuperPos - 1) / kSuperPos);
  if constexpr (PF == 1) {
    read_rows(1);
    Slot pre = step(first_stage{}, pre0, 0);
    for (int st = 1; st < n_st; ++st) pre = step(later_stage{}, pre, st);
  } else {
    read_rows(1);
    Slot pre1 = fetch();
    read_rows(2);
    pre0 = step(first_stage{}, pre0, 0);
    int st = 1;
    for (; st + 2 <= n_st; st += 2) {   // whole rounds (stage st in slot st % 2)
      pre1 = step(later_stage{}, pre1, st);
      pre0 = step(later_stage{}, pre0, st + 1);
    }
    if (st < n_st) step(later_stage{}, pre1, st);
  }
  // the last tile (odd index) is still in set B
  float p0 = 0.f, p1 = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) epi_elem(accB, e, p0, p1);
  epilogue_store(p0, p1, n_st * kSuperTiles - 1);
}

template <int KS16>
dsa_status launch_rows(const void* q, const float* w, const void* kidx, const int32_t* bt, const int32_t* row_len,
                       float* scores, int B, int R, int H, int page, int max_pages, int64_t ld, hipStream_t s) {
  // about DSA_INDEX_ROWS_WGS workgroups per launch, chunks of at most 4096 positions
#ifndef DSA_INDEX_ROWS_WGS
#define DSA_INDEX_ROWS_WGS 512
#endif
  const int64_t tiles = (ld + kRowsTile - 1) / kRowsTile;
  int per = (int)((tiles * B + DSA_INDEX_ROWS_WGS - 1) / DSA_INDEX_ROWS_WGS);
  per = per < 1 ? 1 : per > kMaxChunkPositions / kRowsTile ? kMaxChunkPositions / kRowsTile : per;
  const int chunk = per * kRowsTile;
  dim3 grid((unsigned)((ld + chunk - 1) / chunk), (unsigned)B);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(kidx);
  // up to 4 rows: one wave per row; 5..8 rows: eight waves (rows past R hold
  // zero Q), staged four tiles per barrier and software-pipelined
#define DSA_ROWS_LAUNCH(NW) \
  hipLaunchKernelGGL((index_scores_rows_kernel<KS16, NW>), grid, dim3(NW * 64), 0, s, qq, w, kk, bt, row_len, \
                     scores, R, H, page, max_pages, ld, chunk)
  switch (R) {
    case 2: DSA_ROWS_LAUNCH(2); break;
    case 3: DSA_ROWS_LAUNCH(3); break;
    case 4: DSA_ROWS_LAUNCH(4); break;
    default: {
      // five to eight rows: one workgroup per CU, chunks of whole 128-position stages
      int sp = (int)((tiles * B + DSA_INDEX_SUPER_WGS - 1) / DSA_INDEX_SUPER_WGS);
      sp = (sp + kSuperTiles - 1) / kSuperTiles * kSuperTiles;
      sp = sp > kMaxChunkPositions / kRowsTile ? kMaxChunkPositions / kRowsTile : sp;
      const int schunk = sp * kRowsTile;
      const size_t lds = super_lds_bytes<KS16>();
      auto kern = index_scores_rows8_kernel<KS16>;
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds) != hipSuccess) {
        set_error("dsa_index_scores: %zu bytes of LDS not available", lds);
        return DSA_ERR_HIP;
      }
      hipLaunchKernelGGL(kern, dim3((unsigned)((ld + schunk - 1) / schunk), (unsigned)B), dim3(kSuperThreads), lds, s,
                         qq, w, kk, bt, row_len, scores, R, H, page, max_pages, ld, schunk);
      break;
    }
  }
#undef DSA_ROWS_LAUNCH
  return launch_status("dsa_index_scores");
}

template <int KS>
dsa_status dispatch_mb(int MB, const void* q, const float* w, const void* kidx, const int32_t* bt,
                       const int32_t* row_len, float* scores, int B, int R, int H, int page,
                       int max_pages, int64_t ld, hipStream_t s) {
  switch (MB) {
    case 1: return launch_index<KS, 1>(q, w, kidx, bt, row_len, scores, B, R, H, page, max_pages, ld, s);
    case 2: return launch_index<KS, 2>(q, w, kidx, bt, row_len, scores, B, R, H, page, max_pages, ld, s);
    case 3: return launch_index<KS, 3>(q, w, kidx, bt, row_len, scores, B, R, H, page, max_pages, ld, s);
    default: return launch_index<KS, 4>(q, w, kidx, bt, row_len, scores, B, R, H, page, max_pages, ld, s);
  }
}

}  // namespace
}  // namespace dsa

extern "C" dsa_status dsa_index_scores(const void* q, const float* w, const void* k_index,
                                       const int32_t* block_table, const int32_t* row_len,
                                       float* scores, int B, int R, int H_I, int D_I, int page,
                                       int max_pages, int64_t ld, void* stream) {
  using namespace dsa;
  clear_error();
  DSA_REQUIRE(q && w && k_index && block_table && row_len && scores, DSA_ERR_INVALID_ARG,
              "dsa_index_scores: null pointer argument");
  DSA_REQUIRE(B >= 1 && R >= 1 && H_I >= 1 && D_I >= 1 && page >= 1 && max_pages >= 1 && ld >= 1,
              DSA_ERR_INVALID_ARG, "dsa_index_scores: sizes must be positive (B=%d R=%d H_I=%d D_I=%d page=%d max_pages=%d ld=%lld)",
              B, R, H_I, D_I, page, max_pages, (long long)ld);
  DSA_REQUIRE(D_I == 32 || D_I == 64 || D_I == 128, DSA_ERR_UNSUPPORTED,
              "dsa_index_scores: D_I=%d not in {32, 64, 128}", D_I);
  DSA_REQUIRE(H_I <= 64, DSA_ERR_UNSUPPORTED, "dsa_index_scores: H_I=%d > 64", H_I);
  DSA_REQUIRE(R <= 8, DSA_ERR_UNSUPPORTED, "dsa_index_scores: R=%d > 8", R);
  DSA_REQUIRE(B <= 65535, DSA_ERR_UNSUPPORTED, "dsa_index_scores: B=%d > 65535", B);
  DSA_REQUIRE(ld <= DSA_MAX_LD, DSA_ERR_UNSUPPORTED, "dsa_index_scores: ld=%lld > %lld", (long long)ld,
              (long long)DSA_MAX_LD);
  DSA_REQUIRE(aligned16(q) && aligned16(k_index), DSA_ERR_INVALID_ARG,
              "dsa_index_scores: q and k_index must be 16-byte aligned");
  const int MB = (H_I + 15) / 16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (R >= 2) {   // several query rows: GEMM-shaped kernel, Q fragments in registers
    switch (D_I) {
      case 32: return launch_rows<2>(q, w, k_index, block_table, row_len, scores, B, R, H_I, page, max_pages, ld, s);
      case 64: return launch_rows<4>(q, w, k_index, block_table, row_len, scores, B, R, H_I, page, max_pages, ld, s);
      default: return launch_rows<8>(q, w, k_index, block_table, row_len, scores, B, R, H_I, page, max_pages, ld, s);
    }
  }
  switch (D_I) {
    case 32: return dispatch_mb<1>(MB, q, w, k_index, block_table, row_len, scores, B, R, H_I, page, max_pages, ld, s);
    case 64: return dispatch_mb<2>(MB, q, w, k_index, block_table, row_len, scores, B, R, H_I, page, max_pages, ld, s);
    default: return dispatch_mb<4>(MB, q, w, k_index, block_table, row_len, scores, B, R, H_I, page, max_pages, ld, s);
  }
}
