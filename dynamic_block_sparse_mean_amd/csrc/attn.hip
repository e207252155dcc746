// Block-sparse attention over the kept tiles.
//
// Page "600倍加速，720p视频实时生成！单卡也能带的动14B模型", dynamic sparse quantized
// attention paragraph: only the activated tiles are computed and they are computed densely;
// efficient inference operators paragraph: Q/K in INT8 and V in FP8. Page "Run Wan2.2-A14B
// on One RTX 5090", section 3: dense computation inside the surviving blocks. Readings: no
// causal mask; softmax scale 1/sqrt(d); tiles visited in ascending key-block order; online
// softmax in fp32 in the log2 domain; P scaled by 2^8 and rounded to FP8 E4M3 (RNE) for the
// PV product, the row sum taken from the fp32 P before rounding.
//
// Work split: one workgroup per (batch, head, query block), block_q/32 wavefronts of 32
// query rows each. All wavefronts of a workgroup share the block's kept key list, so every
// kept 64-key sub-tile (K^ 8 KB + V^T 8 KB in INT8/FP8 mode) is copied once into LDS
// (double-buffered) and read by all of them.
//
// Per wavefront and 64-key sub-tile, INT8/FP8 mode:
//   S^T[64 keys][32 queries] = K^ Q^^T : 8 x v_mfma_i32_32x32x32_i8, exact int32.
//     The transposed product leaves each lane with one query row (lane % 32) and 32 of its
//     64 keys (the other 32 in lane ^ 32), so row max and row sum are lane-local but for a
//     single exchange with the partner lane.
//   x = S * g with g = fl(fl(s_q s_k) * fl(sm log2 e)); running max m, alpha = 2^(m - m');
//   p256 = 2^(x - (m' - 8)) = p * 2^8;  l += p256 (fp32, before rounding);
//   P^ = fp8(p256) packed straight from the accumulator registers into the B operand of
//   O^T[128 d][32 q] += V^T P^^T : 4 x v_mfma_f32_32x32x64_f8f6f4 (V^T's key order in memory
//   matches the register order of P, so no shuffle is needed).
//   The per-block V scale is folded into the accumulator's units: before tile j the
//   accumulator is multiplied by alpha * s_v(prev)/s_v(j), and the output is
//   acc * s_v(last) / l at the end (l counted in units of p * 2^8).
#include "sa_internal.h"

namespace sa {

// ---------------------------------------------------------------------------------------
// shared pieces
// ---------------------------------------------------------------------------------------

// Copy `bytes` (multiple of 16 * nthreads) from global to LDS, linear.
template <int NT, int BYTES>
struct TileCopy {
  static constexpr int kPer = BYTES / (16 * NT);
  uint4 r[kPer];
  __device__ __forceinline__ void load(const uint8_t* __restrict__ src, int t) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) r[k] = *(const uint4*)(src + (k * NT + t) * 16);
  }
  __device__ __forceinline__ void store(uint8_t* dst, int t) const {
#pragma unroll
    for (int k = 0; k < kPer; ++k) *(uint4*)(dst + (k * NT + t) * 16) = r[k];
  }
};

// S^T of one 64-key INT8 sub-tile for one wavefront: acc[kb] holds keys 32kb..32kb+31.
// ldsK: [64][128] int8 with the chunk swizzle; qB[c] = Q^ bytes 32c+16g..+15 of query n.
__device__ __forceinline__ void qk_subtile_i8(const uint8_t* ldsK, const v4i qB[4], int n, int g,
                                              v16i acc[2]) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    v16i c0 = {};
    const int row = 32 * kb + n;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int chunk = (2 * c + g) ^ (row & 7);
      const v4i a = *(const v4i*)(ldsK + row * kD + chunk * 16);
      c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qB[c], c0, 0, 0, 0);
    }
    acc[kb] = c0;
  }
}

// Q^ operand of query row `row` (of the block) for lane group g.
__device__ __forceinline__ void load_q_i8(const int8_t* qblk, int row, int g, v4i qB[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) qB[c] = *(const v4i*)(qblk + row * kD + 32 * c + 16 * g);
}

// Key index (0..63 in the sub-tile) held by accumulator register v of block kb, lane group g.
__device__ __forceinline__ int acc_key(int kb, int v, int g) {
  return 32 * kb + 8 * (v >> 2) + 4 * g + (v & 3);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// Write the O^T accumulators of one wavefront (rows of the block) as bf16.
__device__ __forceinline__ void store_out(const v16f acc[4], float scale, __bf16* out, int64_t ol,
                                          int64_t row_global, bool row_ok, int g) {
  if (!row_ok) return;
  __bf16* orow = out + row_global * ol;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * db + 8 * q4 + 4 * g;
      uint2 w;
      w.x = pack_bf16x2(acc[db][4 * q4 + 0] * scale, acc[db][4 * q4 + 1] * scale);
      w.y = pack_bf16x2(acc[db][4 * q4 + 2] * scale, acc[db][4 * q4 + 3] * scale);
      *(uint2*)(orow + d) = w;
    }
}

// ---------------------------------------------------------------------------------------
// INT8 QK^T + FP8 PV
// ---------------------------------------------------------------------------------------
template <int BQ>
__global__ __launch_bounds__(BQ * 2) void attn_i8f8_kernel(
    const int8_t* __restrict__ Qh, const uint8_t* __restrict__ Kh, const uint8_t* __restrict__ Vt,
    const float* __restrict__ sq, const float* __restrict__ sk, const float* __restrict__ sv,
    const int32_t* __restrict__ plan, int64_t H, int64_t L, int64_t nQ, int64_t nK, int nsub,
    int64_t n_keep, float c_log2, __bf16* __restrict__ out, int64_t ob, int64_t oh, int64_t ol,
    int64_t total) {
  constexpr int NT = BQ * 2;
  constexpr int kTile = 2 * 64 * kD;  // K^ + V^T bytes of a sub-tile
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kTile];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63, n = lane & 31, g = lane >> 5;
  const int64_t w = xcd_remap(blockIdx.x, total);
  const int64_t bh = w / nQ, i = w % nQ;
  const int64_t b = bh / H, h = bh % H;
  const int32_t* prow = plan + (bh * nQ + i) * n_keep;
  const int64_t U = n_keep * nsub;
  const int bk = 64 * nsub;

  v4i qB[4];
  load_q_i8(Qh + (bh * nQ + i) * (int64_t)BQ * kD, 32 * wave + n, g, qB);
  const float s_q = sq[bh * nQ + i];

  float m = -INFINITY, l = 0.f, units = 1.f;
  v16f acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = (v16f){};

  auto tile_src = [&](int64_t u, int64_t& j, int& s, bool& ok) -> int64_t {
    j = prow[u / nsub];
    s = (int)(u % nsub);
    ok = j >= 0 && j < nK;
    const int64_t jj = ok ? j : 0;
    return ((bh * nK + jj) * nsub + s) * (int64_t)(64 * kD);
  };

  TileCopy<NT, 64 * kD> ck, cv;
  {
    int64_t j; int s; bool ok;
    const int64_t off = tile_src(0, j, s, ok);
    ck.load(Kh + off, t);
    cv.load(Vt + off, t);
    ck.store(lds[0], t);
    cv.store(lds[0] + 64 * kD, t);
  }
  __syncthreads();

  for (int64_t u = 0; u < U; ++u) {
    const int st = (int)(u & 1);
    if (u + 1 < U) {
      int64_t j1; int s1; bool ok1;
      const int64_t off = tile_src(u + 1, j1, s1, ok1);
      ck.load(Kh + off, t);
      cv.load(Vt + off, t);
    }
    int64_t j; int s; bool ok;
    tile_src(u, j, s, ok);
    const int64_t key0 = j * bk + 64 * s;
    const int valid = ok ? (int)((L - key0) < 64 ? (L - key0) : 64) : 0;
    if (valid > 0) {
      const uint8_t* ldsK = lds[st];
      const uint8_t* ldsV = lds[st] + 64 * kD;
      v16i S[2];
      qk_subtile_i8(ldsK, qB, n, g, S);
      const float gt = (s_q * sk[bh * nK + j]) * c_log2;
      const float svj = sv[bh * nK + j];
      int mx = INT_MIN;
      if (valid == 64) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = max(mx, S[kb][v]);
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (acc_key(kb, v, g) < valid) mx = max(mx, S[kb][v]);
      }
      mx = max(mx, __shfl_xor(mx, 32, 64));
      const float xmax = mx == INT_MIN ? -INFINITY : (float)mx * gt;
      const float m_new = fmaxf(m, xmax);
      const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
      const float u_new = svj > 0.f ? svj : units;
      const float factor = m == -INFINITY ? 0.f : alpha * (units / u_new);
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] *= factor;
      const float mb = m_new - 8.f;
      float lsum = 0.f;
      v8i P;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; v += 4) {
          float p[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float y = __builtin_fmaf((float)S[kb][v + e], gt, -mb);
            p[e] = __builtin_amdgcn_exp2f(y);
            if (valid < 64 && acc_key(kb, v + e, g) >= valid) p[e] = 0.f;
            lsum += p[e];
          }
          int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
          wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wd, true);
          P[4 * kb + (v >> 2)] = wd;
        }
      l = alpha * l + lsum;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = 32 * db + n;
        const int sw = (d >> 1) & 3;
        const uint8_t* rowp = ldsV + d * 64;
        const v4i lo = *(const v4i*)(rowp + (((2 * g) ^ sw) << 4));
        const v4i hi = *(const v4i*)(rowp + (((2 * g + 1) ^ sw) << 4));
        const v8i a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, P, acc[db], 0, 0, 0, 0, 0, 0);
      }
      m = m_new;
      units = u_new;
    }
    if (u + 1 < U) {
      ck.store(lds[st ^ 1], t);
      cv.store(lds[st ^ 1] + 64 * kD, t);
    }
    __syncthreads();
  }
  const float l_tot = l + __shfl_xor(l, 32, 64);
  const float scale = units / l_tot;
  const int64_t row = i * BQ + 32 * wave + n;
  store_out(acc, scale, out + b * ob + h * oh, ol, row, row < L, g);
}

// Debug: the int32 S tile of query block i against key block plan[prow_off] through
// qk_subtile_i8 (the attention kernel's own MFMA path). An index outside [0, nK) reads block 0.
template <int BQ>
__global__ __launch_bounds__(BQ * 2) void debug_qk_kernel(const int8_t* __restrict__ Qh,
                                                          const uint8_t* __restrict__ Kh,
                                                          const int32_t* __restrict__ plan,
                                                          int64_t prow_off, int64_t nQ, int64_t nK,
                                                          int nsub, int64_t bh, int64_t i,
                                                          int32_t* __restrict__ out) {
  constexpr int NT = BQ * 2;
  __shared__ __attribute__((aligned(16))) uint8_t ldsK[64 * kD];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63, n = lane & 31, g = lane >> 5;
  int64_t j = plan[prow_off];
  if (j < 0 || j >= nK) j = 0;
  v4i qB[4];
  load_q_i8(Qh + (bh * nQ + i) * (int64_t)BQ * kD, 32 * wave + n, g, qB);
  for (int s = 0; s < nsub; ++s) {
    TileCopy<NT, 64 * kD> ck;
    ck.load(Kh + ((bh * nK + j) * nsub + s) * (int64_t)(64 * kD), t);
    __syncthreads();
    ck.store(ldsK, t);
    __syncthreads();
    v16i S[2];
    qk_subtile_i8(ldsK, qB, n, g, S);
    const int q = 32 * wave + n;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) out[q * (64 * nsub) + 64 * s + acc_key(kb, v, g)] = S[kb][v];
  }
}

// ---------------------------------------------------------------------------------------
// BF16 QK^T + BF16 PV (no quantization)
// ---------------------------------------------------------------------------------------
template <int BQ>
__global__ __launch_bounds__(BQ * 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, int64_t qsb, int64_t qsh, int64_t qsl,
    const uint8_t* __restrict__ Kt, const uint8_t* __restrict__ Vt, const int32_t* __restrict__ plan,
    int64_t H, int64_t L, int64_t nQ, int64_t nK, int nsub, int64_t n_keep, float c_log2,
    __bf16* __restrict__ out, int64_t ob, int64_t oh, int64_t ol, int64_t total) {
  constexpr int NT = BQ * 2;
  constexpr int kHalf = 64 * kD * 2;  // K or V^T bytes of a bf16 sub-tile
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2 * kHalf];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63, n = lane & 31, g = lane >> 5;
  const int64_t w = xcd_remap(blockIdx.x, total);
  const int64_t bh = w / nQ, i = w % nQ;
  const int64_t b = bh / H, h = bh % H;
  const int32_t* prow = plan + (bh * nQ + i) * n_keep;
  const int64_t U = n_keep * nsub;
  const int bk = 64 * nsub;

  // Q operand: 8 chunks of 8 bf16 (d = 16c + 8g ..) of query row `row`.
  v8bf qB[8];
  const int64_t row = i * BQ + 32 * wave + n;
  {
    const uint16_t* qrow = q + b * qsb + h * qsh + (row < L ? row : 0) * qsl;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint4 r = make_uint4(0, 0, 0, 0);
      if (row < L) r = *(const uint4*)(qrow + 16 * c + 8 * g);
      qB[c] = __builtin_bit_cast(v8bf, r);
    }
  }
  float m = -INFINITY, l = 0.f;
  v16f acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = (v16f){};

  auto tile_src = [&](int64_t u, int64_t& j, int& s, bool& ok) -> int64_t {
    j = prow[u / nsub];
    s = (int)(u % nsub);
    ok = j >= 0 && j < nK;
    const int64_t jj = ok ? j : 0;
    return ((bh * nK + jj) * nsub + s) * (int64_t)kHalf;
  };

  TileCopy<NT, kHalf> ck, cv;
  {
    int64_t j; int s; bool ok;
    const int64_t off = tile_src(0, j, s, ok);
    ck.load(Kt + off, t);
    cv.load(Vt + off, t);
    ck.store(lds[0], t);
    cv.store(lds[0] + kHalf, t);
  }
  __syncthreads();

  for (int64_t u = 0; u < U; ++u) {
    const int st = (int)(u & 1);
    if (u + 1 < U) {
      int64_t j1; int s1; bool ok1;
      const int64_t off = tile_src(u + 1, j1, s1, ok1);
      ck.load(Kt + off, t);
      cv.load(Vt + off, t);
    }
    int64_t j; int s; bool ok;
    tile_src(u, j, s, ok);
    const int64_t key0 = j * bk + 64 * s;
    const int valid = ok ? (int)((L - key0) < 64 ? (L - key0) : 64) : 0;
    if (valid > 0) {
      const uint8_t* ldsK = lds[st];
      const uint8_t* ldsV = lds[st] + kHalf;
      v16f S[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        v16f c0 = {};
        const int r = 32 * kb + n;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int chunk = (2 * c + g) ^ (r & 7);
          const v8bf a = *(const v8bf*)(ldsK + r * (kD * 2) + chunk * 16);
          c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qB[c], c0, 0, 0, 0);
        }
        S[kb] = c0;
      }
      float smax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          if (valid < 64 && acc_key(kb, v, g) >= valid) S[kb][v] = -INFINITY;
          smax = fmaxf(smax, S[kb][v]);
        }
      smax = fmaxf(smax, __shfl_xor(smax, 32, 64));
      const float m_new = fmaxf(m, smax * c_log2);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 while m = -inf
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] *= alpha;
      }
      float lsum = 0.f;
      v8bf P[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint32_t wd[4];
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][8 * hh + e], c_log2, -m_new));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][8 * hh + e + 1], c_log2, -m_new));
            lsum += p0 + p1;
            wd[e >> 1] = pack_bf16x2(p0, p1);
          }
          P[2 * kb + hh] = __builtin_bit_cast(v8bf, make_uint4(wd[0], wd[1], wd[2], wd[3]));
        }
      l = alpha * l + lsum;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = 32 * db + n;
        const uint8_t* rowp = ldsV + d * (64 * 2);
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const int chunk = (2 * kc + g) ^ (d & 7);
          const v8bf a = *(const v8bf*)(rowp + chunk * 16);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, P[kc], acc[db], 0, 0, 0);
        }
      }
      m = m_new;
    }
    if (u + 1 < U) {
      ck.store(lds[st ^ 1], t);
      cv.store(lds[st ^ 1] + kHalf, t);
    }
    __syncthreads();
  }
  const float l_tot = l + __shfl_xor(l, 32, 64);
  store_out(acc, 1.f / l_tot, out + b * ob + h * oh, ol, row, row < L, g);
}

// ---------------------------------------------------------------------------------------
void launch_attend_i8f8(const sa_forward_layout& lay, const char* ws, const int32_t* plan,
                        int64_t B, int64_t H, int64_t L, int bq, int bk, int64_t n_keep,
                        float c_log2, const TensorView& out, hipStream_t s) {
  const int64_t total = B * H * lay.nQ;
  const int nsub = bk / 64;
  const int8_t* Qh = (const int8_t*)(ws + lay.q_off);
  const uint8_t* Kh = (const uint8_t*)(ws + lay.k_off);
  const uint8_t* Vt = (const uint8_t*)(ws + lay.v_off);
  const float* sq = (const float*)(ws + lay.sq_off);
  const float* sk = (const float*)(ws + lay.sk_off);
  const float* sv = (const float*)(ws + lay.sv_off);
  __bf16* o = (__bf16*)out.data;
  if (bq == 128)
    attn_i8f8_kernel<128><<<(unsigned)total, 256, 0, s>>>(Qh, Kh, Vt, sq, sk, sv, plan, H, L, lay.nQ,
                                                          lay.nK, nsub, n_keep, c_log2, o, out.sb,
                                                          out.sh, out.sl, total);
  else
    attn_i8f8_kernel<64><<<(unsigned)total, 128, 0, s>>>(Qh, Kh, Vt, sq, sk, sv, plan, H, L, lay.nQ,
                                                         lay.nK, nsub, n_keep, c_log2, o, out.sb,
                                                         out.sh, out.sl, total);
}

void launch_attend_bf16(const TensorView& q, const sa_forward_layout& lay, const char* ws,
                        const int32_t* plan, int64_t B, int64_t H, int64_t L, int bq, int bk,
                        int64_t n_keep, float c_log2, const TensorView& out, hipStream_t s) {
  const int64_t total = B * H * lay.nQ;
  const int nsub = bk / 64;
  const uint8_t* Kt = (const uint8_t*)(ws + lay.k_off);
  const uint8_t* Vt = (const uint8_t*)(ws + lay.v_off);
  __bf16* o = (__bf16*)out.data;
  if (bq == 128)
    attn_bf16_kernel<128><<<(unsigned)total, 256, 0, s>>>((const uint16_t*)q.data, q.sb, q.sh, q.sl, Kt,
                                                          Vt, plan, H, L, lay.nQ, lay.nK, nsub,
                                                          n_keep, c_log2, o, out.sb, out.sh, out.sl,
                                                          total);
  else
    attn_bf16_kernel<64><<<(unsigned)total, 128, 0, s>>>((const uint16_t*)q.data, q.sb, q.sh, q.sl, Kt,
                                                         Vt, plan, H, L, lay.nQ, lay.nK, nsub,
                                                         n_keep, c_log2, o, out.sb, out.sh, out.sl,
                                                         total);
}

void launch_debug_qk(const sa_forward_layout& lay, const char* ws, const int32_t* plan, int64_t B,
                     int64_t H, int64_t L, int bq, int bk, int64_t n_keep, int64_t b, int64_t h,
                     int64_t i, int64_t t, int32_t* out, hipStream_t s) {
  (void)B; (void)L;
  const int nsub = bk / 64;
  const int64_t prow_off = ((b * H + h) * lay.nQ + i) * n_keep + t;
  const int8_t* Qh = (const int8_t*)(ws + lay.q_off);
  const uint8_t* Kh = (const uint8_t*)(ws + lay.k_off);
  if (bq == 128)
    debug_qk_kernel<128><<<1, 256, 0, s>>>(Qh, Kh, plan, prow_off, lay.nQ, lay.nK, nsub, b * H + h, i, out);
  else
    debug_qk_kernel<64><<<1, 128, 0, s>>>(Qh, Kh, plan, prow_off, lay.nQ, lay.nK, nsub, b * H + h, i, out);
}

}  // namespace sa
