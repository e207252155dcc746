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
#include "sa_internal.h"

namespace sa {

// ---------------------------------------------------------------------------
// scores[bh][i][j] = sum_d qm[bh][i][d] * km[bh][j][d]   (fp64, 64 x 64 tile per workgroup)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void scores_kernel(const double* __restrict__ qm,
                                                     const double* __restrict__ km, int64_t nQ,
                                                     int64_t nK, double* __restrict__ S) {
  constexpr int T = 64, DC = 32;
  __shared__ double qs[DC][T + 1];
  __shared__ double ks[DC][T + 1];
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  const int64_t j0 = (int64_t)blockIdx.x * T, i0 = (int64_t)blockIdx.y * T, bh = blockIdx.z;
  const double* qb = qm + bh * nQ * kD;
  const double* kb = km + bh * nK * kD;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = 0.0;
  const int lr = t >> 2, ld = (t & 3) * 8;  // loader: row, first d of 8
  for (int d0 = 0; d0 < kD; d0 += DC) {
    {
      const int64_t qi = i0 + lr, kj = j0 + lr;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qs[ld + e][lr] = qi < nQ ? qb[qi * kD + d0 + ld + e] : 0.0;
        ks[ld + e][lr] = kj < nK ? kb[kj * kD + d0 + ld + e] : 0.0;
      }
    }
    __syncthreads();
#pragma unroll 8
    for (int d = 0; d < DC; ++d) {
      double qa[4], kc[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) qa[a] = qs[d][ty + 16 * a];
#pragma unroll
      for (int c = 0; c < 4; ++c) kc[c] = ks[d][tx + 16 * c];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = fma(qa[a], kc[c], acc[a][c]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t i = i0 + ty + 16 * a;
    if (i >= nQ) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t j = j0 + tx + 16 * c;
      if (j < nK) S[(bh * nQ + i) * nK + j] = acc[a][c];
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

// Lane l holds the contiguous index range [l*chunk, l*chunk + chunk) of the row, slot c
// is index l*chunk + c. Candidates narrow pass by pass through a 256-bin histogram:
// first over the value range [lo, hi] of the candidates (scores are spread over the bins,
// so the LDS counters see little contention), then, if a row has not resolved after
// kValuePasses, over the bytes of an order-preserving 64-bit key (at most 8 passes).
// Whatever remains is a set of equal scores, taken in index order.
template <int MAXC>
__global__ __launch_bounds__(64) void topk_kernel(const double* __restrict__ S, int64_t nK,
                                                  int64_t n_keep, int32_t* __restrict__ plan) {
  constexpr int kValuePasses = 12;
  __shared__ int hist[256];
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const int chunk = (int)((nK + 63) / 64);
  const int64_t j0 = (int64_t)lane * chunk;
  const double* s = S + row * nK;
  double v[MAXC];
  uint64_t cand = 0, sel = 0;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int64_t j = j0 + c;
    const bool ok = c < chunk && j < nK;
    v[c] = ok ? s[j] : 0.0;
    if (ok) cand |= (1ull << c);
  }
  int64_t k = n_keep;
  bool done = false;
  for (int pass = 0; pass < kValuePasses + 8 && !done; ++pass) {
    const int ncand = wave_sum_i32(__popcll(cand));
    if (ncand == k) {  // every remaining candidate is needed
      sel |= cand;
      cand = 0;
      done = true;
      break;
    }
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
    for (int e = lane; e < 256; e += 64) hist[e] = 0;
    __syncthreads();
    int bins[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      int bin;
      if (value_mode) {
        bin = (int)((v[c] - lo) * scale);
        bin = bin > 255 ? 255 : (bin < 0 ? 0 : bin);
      } else {
        bin = (int)((order_key(v[c]) >> shift) & 255);
      }
      bins[c] = bin;
      if (cand >> c & 1) atomicAdd(&hist[bin], 1);
    }
    __syncthreads();
    // Lane l owns bins 4l..4l+3. Count of candidates in bins above each of them.
    const int h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
              h3 = hist[4 * lane + 3];
    const int local = h0 + h1 + h2 + h3;
    const int excl = wave_excl_scan_i32(local, lane);
    const int total = __shfl(excl + local, 63, 64);
    const int above_lane = total - excl - local;  // in bins of higher lanes
    int found = -1, cnt_above = 0, cnt_bin = 0;
    {
      const int hb[4] = {h0, h1, h2, h3};
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
      if (bins[c] > bstar) sel |= (1ull << c);
      if (bins[c] != bstar) cand &= ~(1ull << c);
    }
    k -= above;
    if (inbin == k) {
      sel |= cand;
      cand = 0;
      done = true;
    }
    __syncthreads();
  }
  if (!done) {
    // Remaining candidates hold equal scores: the lowest indices win.
    const int mine = __popcll(cand);
    int rank = wave_excl_scan_i32(mine, lane);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      if (cand >> c & 1) {
        if (rank < k) sel |= (1ull << c);
        ++rank;
      }
    }
  }
  const int nsel = __popcll(sel);
  int pos = wave_excl_scan_i32(nsel, lane);
  int32_t* out = plan + row * n_keep;
#pragma unroll
  for (int c = 0; c < MAXC; ++c)
    if (sel >> c & 1) {
      if (pos < n_keep) out[pos] = (int32_t)(j0 + c);
      ++pos;
    }
}

void launch_scores(const double* qm, const double* km, int64_t BH, int64_t nQ, int64_t nK,
                   double* scores, hipStream_t s) {
  const dim3 grid((unsigned)((nK + 63) / 64), (unsigned)((nQ + 63) / 64), (unsigned)BH);
  scores_kernel<<<grid, 256, 0, s>>>(qm, km, nQ, nK, scores);
}

void launch_topk(const double* scores, int64_t rows, int64_t nK, int64_t n_keep, int32_t* plan,
                 hipStream_t s) {
  const int64_t chunk = (nK + 63) / 64;
  const dim3 grid((unsigned)rows);
  if (chunk <= 8) topk_kernel<8><<<grid, 64, 0, s>>>(scores, nK, n_keep, plan);
  else if (chunk <= 16) topk_kernel<16><<<grid, 64, 0, s>>>(scores, nK, n_keep, plan);
  else if (chunk <= 32) topk_kernel<32><<<grid, 64, 0, s>>>(scores, nK, n_keep, plan);
  else topk_kernel<64><<<grid, 64, 0, s>>>(scores, nK, n_keep, plan);
}

}  // namespace sa
