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
#include "dsa_common.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;      // 4 waves

// TILES 16-position MFMA N tiles per wave step; a workgroup step covers
// 4 * 16 * TILES positions.
template <int KS, int MB, int TILES>
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
  for (int r = 0; r < R; ++r) lmax = max(lmax, row_len[b * R + r]);
  const int t_begin = blockIdx.x * chunk;
  if (t_begin >= lmax) return;  // uniform across the workgroup
  const int t_end = min(t_begin + chunk, lmax);
  const int n_iter = (t_end - t_begin + kBlockPos - 1) / kBlockPos;   // >= 1, same for every wave

  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int32_t* bt = block_table + (size_t)b * max_pages;

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
      const int phys = bt[t / page];
      const uint16_t* src = kidx + ((size_t)phys * page + (t % page)) * D + g * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bf[tile][ks] = *reinterpret_cast<const bf16x8_t*>(src + ks * 32);
    }
    if (it == 0) {
      // Q fragments in A-operand order (issued after the first key loads so
      // the two round trips overlap): fragment (r, mb, ks), lane l holds head
      // mb*16 + l%16, dims ks*32 + (l/16)*8 .. +8.  Heads >= H are zero.
      const int nfrag = R * MB * KS * 64;
      for (int i = tid; i < nfrag; i += kThreads) {
        const int fl = i & 63;
        const int f = i >> 6;
        const int ks = f % KS;
        const int mb = (f / KS) % MB;
        const int r = f / (KS * MB);
        const int h = mb * 16 + (fl & 15);
        bf16x8_t v = {};
        if (h < H) {
          const uint16_t* src = q + ((size_t)(b * R + r) * H + h) * D + ks * 32 + (fl >> 4) * 8;
          v = *reinterpret_cast<const bf16x8_t*>(src);
        }
        qs[i] = v;
      }
      for (int i = tid; i < R * MB * 16; i += kThreads) {
        const int r = i / (MB * 16);
        const int h = i % (MB * 16);
        wl[i] = h < H ? w[(size_t)(b * R + r) * H + h] : 0.f;
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
      if (g < TILES && t < t_end && t < row_len[b * R + r]) scores[(size_t)(b * R + r) * ld + t] = mine;
    }
  }
}

template <int KS, int MB, int TILES>
dsa_status launch_index_t(const void* q, const float* w, const void* kidx, const int32_t* bt,
                          const int32_t* row_len, float* scores, int B, int R, int H, int page,
                          int max_pages, int64_t ld, hipStream_t stream) {
  constexpr int kBlockPos = kThreads / 64 * 16 * TILES;
  const size_t lds = (size_t)R * MB * KS * 64 * 16 + (size_t)R * MB * 16 * sizeof(float);
  auto kern = index_scores_kernel<KS, MB, TILES>;
  if (lds > 65536) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
      set_error("dsa_index_scores: %zu bytes of LDS not available", lds);
      return DSA_ERR_UNSUPPORTED;
    }
  }
  // Positions per workgroup: whole steps, sized so that a long row still
  // spreads over about 2048 workgroups.
  const int64_t steps = (ld + kBlockPos - 1) / kBlockPos;
  int per = (int)((steps * B + 2047) / 2048);
  per = per < 1 ? 1 : per > 8 ? 8 : per;
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
  // small problems: one 16-position tile per wave step, so more workgroups
  const int64_t total = ld * (int64_t)B;
  if (total <= (1 << 18))
    return launch_index_t<KS, MB, 1>(q, w, kidx, bt, row_len, scores, B, R, H, page, max_pages, ld, stream);
  if (total <= (1 << 20))
    return launch_index_t<KS, MB, 2>(q, w, kidx, bt, row_len, scores, B, R, H, page, max_pages, ld, stream);
  return launch_index_t<KS, MB, 4>(q, w, kidx, bt, row_len, scores, B, R, H, page, max_pages, ld, stream);
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
  DSA_REQUIRE(ld <= ((int64_t)1 << 31) - 1, DSA_ERR_UNSUPPORTED, "dsa_index_scores: ld too large");
  DSA_REQUIRE(aligned16(q) && aligned16(k_index), DSA_ERR_INVALID_ARG,
              "dsa_index_scores: q and k_index must be 16-byte aligned");
  const int MB = (H_I + 15) / 16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (D_I) {
    case 32: return dispatch_mb<1>(MB, q, w, k_index, block_table, row_len, scores, B, R, H_I, page, max_pages, ld, s);
    case 64: return dispatch_mb<2>(MB, q, w, k_index, block_table, row_len, scores, B, R, H_I, page, max_pages, ld, s);
    default: return dispatch_mb<4>(MB, q, w, k_index, block_table, row_len, scores, B, R, H_I, page, max_pages, ld, s);
  }
}
