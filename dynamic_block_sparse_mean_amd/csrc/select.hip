// Pooled scores and per-row top-k: the run-time choice of key blocks.
//
// Page "600倍加速，720p视频实时生成！单卡也能带的动14B模型": the block means estimate how
// important each attention tile is, then the important key blocks are picked at run time
// (dynamic sparse quantized attention paragraph), judged from the current Q/K (efficient
// inference operators paragraph). Readings: score = Qbar_i . Kbar_j in fp64; each query
// block keeps its n_keep highest scores, equal scores go to the lower block index, and the
// kept indices are written in ascending order.
//
// Two kernels: a tiled fp64 product Qbar Kbar^T per (batch, head) writing the score matrix
// to the workspace, then one wavefront per query-block row that selects the top n_keep.
#include <type_traits>

#include "sa_internal.h"

namespace sa {

// ---------------------------------------------------------------------------
// scores[bh][i][j] = sum_d qm[bh][i][d] * km[bh][j][d]   (fp64 MFMA, 64 x 64 tile per workgroup)
// ---------------------------------------------------------------------------
// One workgroup per 64 x 64 tile, the tiles taken in (head, query tile, key tile) order with
// each XCD given a contiguous range of them, so an XCD's workgroups reuse one head's means
// from its L2 instead of every XCD fetching every head's.
// Four wavefronts, each a 32 x 32 quarter of the tile as 2 x 2 v_mfma_f64_16x16x4 blocks. The
// head dimension is staged through LDS 32 values at a time, the next chunk prefetched into
// registers while the current one is multiplied; consecutive threads load consecutive 16-byte
// pieces of the rows, so each load instruction reads 1 KB of contiguous memory. The order in
// which an MFMA consumes d does not matter to the result beyond rounding, so at step s of a
// chunk lane group g (lanes 16g..16g+15) supplies d = 8g + s for both operands: each lane then
// reads 8 consecutive doubles of one row. Rows are padded to 272 bytes so the 16 rows read
// together fall in distinct LDS banks.
typedef double v4d __attribute__((ext_vector_type(4)));

constexpr int kScoreTile = 64, kScoreChunk = 32;

__global__ __launch_bounds__(256) void scores_kernel(const double* __restrict__ qm,
                                                     const double* __restrict__ km, int64_t nQ,
                                                     int64_t nK, double* __restrict__ S, int64_t tiles_i,
                                                     int64_t tiles_j, int64_t total) {
  constexpr int T = kScoreTile, DC = kScoreChunk, kRow = DC + 2;  // row stride in doubles (272 B)
  constexpr int H2 = DC / 2;            // 16-byte pieces per staged row
  constexpr int NP = T * H2 / 256;      // pieces per thread and operand
  __shared__ __attribute__((aligned(16))) double qs[T * kRow];
  __shared__ __attribute__((aligned(16))) double ks[T * kRow];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63, m = lane & 15, g = lane >> 4;
  const int64_t w = xcd_remap(blockIdx.x, total);
  const int64_t per_head = tiles_i * tiles_j, bh = w / per_head, rem = w % per_head;
  const int64_t i0 = rem / tiles_j * T, j0 = rem % tiles_j * T;
  const double* qb = qm + bh * nQ * kD;
  const double* kb = km + bh * nK * kD;
  double2 rq[NP], rk[NP];
  auto fetch = [&](int d0) {  // piece e of thread t: row (t + 256 e) / H2, piece (t + 256 e) % H2
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      const int idx = t + 256 * e, r = idx / H2, c = idx % H2;
      rq[e] = i0 + r < nQ ? *(const double2*)(qb + (i0 + r) * kD + d0 + 2 * c) : make_double2(0.0, 0.0);
      rk[e] = j0 + r < nK ? *(const double2*)(kb + (j0 + r) * kD + d0 + 2 * c) : make_double2(0.0, 0.0);
    }
  };
  const int wr = 32 * (wave >> 1), wc = 32 * (wave & 1);  // quarter of the tile
  v4d acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[a][c] = (v4d){0.0, 0.0, 0.0, 0.0};
  fetch(0);
  for (int d0 = 0; d0 < kD; d0 += DC) {
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      const int idx = t + 256 * e, r = idx / H2, c = idx % H2;
      *(double2*)&qs[r * kRow + 2 * c] = rq[e];
      *(double2*)&ks[r * kRow + 2 * c] = rk[e];
    }
    __syncthreads();
    if (d0 + DC < kD) fetch(d0 + DC);
#pragma unroll
    for (int s2 = 0; s2 < DC / 4; s2 += 2) {
      double2 av[2], bv[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) av[a] = *(const double2*)&qs[(wr + 16 * a + m) * kRow + 8 * g + s2];
#pragma unroll
      for (int c = 0; c < 2; ++c) bv[c] = *(const double2*)&ks[(wc + 16 * c + m) * kRow + 8 * g + s2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a].x, bv[c].x, acc[a][c], 0, 0, 0);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a].y, bv[c].y, acc[a][c], 0, 0, 0);
    }
    __syncthreads();
  }
  // D layout of the f64 16 x 16 block: register r of a lane holds row lane / 16 + 4 r, column
  // lane % 16.
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t i = i0 + wr + 16 * a + g + 4 * r;
      if (i >= nQ) continue;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int64_t j = j0 + wc + 16 * c + m;
        if (j < nK) S[(bh * nQ + i) * nK + j] = acc[a][c][r];
      }
    }
}

// ---------------------------------------------------------------------------
// top-k of one score row per wavefront
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t order_key(double v) {
  // Unsigned key that orders like the value (+0 and -0 map to the same key).
  if (v == 0.0) v = 0.0;
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Slot c of lane l holds index j = 64 c + l of the row (coalesced loads; index order is slot
// order, then lane order). Candidates narrow pass by pass through a 256-bin histogram: first
// over the value range [lo, hi] of the candidates (scores spread over the bins, so the LDS
// counters see little contention; the binning is monotone in the score, so any range is
// correct and a good one only converges faster), then, if a row has not resolved after
// kValuePasses, over the bytes of an order-preserving 64-bit key (at most 8 passes).
// Whatever remains is a set of equal scores, taken in index order.
template <int MAXC>
struct SlotMask {
  typedef typename std::conditional<(MAXC > 32), uint64_t, uint32_t>::type type;
};

__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

template <int MAXC>
__global__ __launch_bounds__(64) void topk_kernel(const double* __restrict__ S, int64_t nK,
                                                  int64_t n_keep, int32_t* __restrict__ plan) {
  typedef typename SlotMask<MAXC>::type mask_t;
  constexpr int kValuePasses = 12;
  __shared__ __attribute__((aligned(16))) int hist[256];
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const double* s = S + row * nK;
  double v[MAXC];
  mask_t cand = 0, sel = 0;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int64_t j = 64 * c + lane;
    const bool ok = j < nK;
    v[c] = ok ? s[j] : 0.0;
    if (ok) cand |= ((mask_t)1 << c);
  }
  int64_t k = n_keep;
  bool done = nK == k;
  if (done) {
    sel = cand;
    cand = 0;
  }
  for (int pass = 0; pass < kValuePasses + 8 && !done; ++pass) {
    const bool value_mode = pass < kValuePasses;
    double lo = INFINITY, hi = -INFINITY;
    if (value_mode) {
#pragma unroll
      for (int c = 0; c < MAXC; ++c)
        if (cand >> c & 1) { lo = fmin(lo, v[c]); hi = fmax(hi, v[c]); }
      lo = wave_min_f64(lo);
      hi = wave_max_f64(hi);
      if (!(hi > lo)) break;  // all candidates equal: ties by index below
    }
    const double scale = value_mode ? 256.0 / (hi - lo) : 0.0;
    const int shift = value_mode ? 0 : 56 - 8 * (pass - kValuePasses);
    auto bin_of = [&](double x) -> int {
      if (value_mode) {
        const int b = (int)((x - lo) * scale);
        return b > 255 ? 255 : (b < 0 ? 0 : b);
      }
      return (int)((order_key(x) >> shift) & 255);
    };
    for (int e = lane; e < 256; e += 64) hist[e] = 0;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (cand >> c & 1) atomicAdd(&hist[bin_of(v[c])], 1);
    __syncthreads();
    // Lane l owns bins 4l..4l+3. Count of candidates in bins above each of them.
    const int4 h4 = *(const int4*)&hist[4 * lane];
    const int local = h4.x + h4.y + h4.z + h4.w;
    const int excl = wave_excl_scan_i32(local, lane);
    const int total = __shfl(excl + local, 63, 64);
    const int above_lane = total - excl - local;  // in bins of higher lanes
    int found = -1, cnt_above = 0, cnt_bin = 0;
    {
      const int hb[4] = {h4.x, h4.y, h4.z, h4.w};
      int cum = above_lane;
#pragma unroll
      for (int bb = 3; bb >= 0; --bb) {
        if (found < 0 && cum < k && k <= cum + hb[bb]) {
          found = 4 * lane + bb;
          cnt_above = cum;
          cnt_bin = hb[bb];
        }
        cum += hb[bb];
      }
    }
    const uint64_t who = __ballot(found >= 0);
    const int src = __ffsll((unsigned long long)who) - 1;
    const int bstar = __shfl(found, src, 64);
    const int above = __shfl(cnt_above, src, 64);
    const int inbin = __shfl(cnt_bin, src, 64);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      if (!(cand >> c & 1)) continue;
      const int b = bin_of(v[c]);
      if (b > bstar) sel |= ((mask_t)1 << c);
      if (b != bstar) cand &= ~((mask_t)1 << c);
    }
    k -= above;
    if (inbin == k) {
      sel |= cand;
      cand = 0;
      done = true;
    }
    __syncthreads();
  }
  const uint64_t below = lanes_below(lane);
  if (!done) {
    // Remaining candidates hold equal scores: the lowest indices win.
    int rank = 0;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const uint64_t m = __ballot(cand >> c & 1);
      if ((cand >> c & 1) && rank + __popcll(m & below) < k) sel |= ((mask_t)1 << c);
      rank += __popcll(m);
    }
  }
  int32_t* out = plan + row * n_keep;
  int base = 0;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const uint64_t m = __ballot(sel >> c & 1);
    const int pos = base + __popcll(m & below);
    if ((sel >> c & 1) && pos < n_keep) out[pos] = 64 * c + lane;
    base += __popcll(m);
  }
}

void launch_scores(const double* qm, const double* km, int64_t BH, int64_t nQ, int64_t nK,
                   double* scores, hipStream_t s) {
  const int64_t tiles_j = (nK + kScoreTile - 1) / kScoreTile, tiles_i = (nQ + kScoreTile - 1) / kScoreTile;
  const int64_t total = BH * tiles_i * tiles_j;
  scores_kernel<<<dim3((unsigned)total), 256, 0, s>>>(qm, km, nQ, nK, scores, tiles_i, tiles_j, total);
}

void launch_topk(const double* scores, int64_t rows, int64_t nK, int64_t n_keep, int32_t* plan,
                 hipStream_t s) {
  const int64_t slots = (nK + 63) / 64;  // nK <= kMaxKeyBlocks = 64 * 64
  const dim3 grid((unsigned)rows);
  if (slots <= 8) topk_kernel<8><<<grid, 64, 0, s>>>(scores, nK, n_keep, plan);
  else if (slots <= 16) topk_kernel<16><<<grid, 64, 0, s>>>(scores, nK, n_keep, plan);
  else if (slots <= 24) topk_kernel<24><<<grid, 64, 0, s>>>(scores, nK, n_keep, plan);
  else if (slots <= 32) topk_kernel<32><<<grid, 64, 0, s>>>(scores, nK, n_keep, plan);
  else topk_kernel<64><<<grid, 64, 0, s>>>(scores, nK, n_keep, plan);
}

}  // namespace sa
