// Operand preparation for the attention kernels.
//
// INT8/FP8 mode - page "600倍加速，720p视频实时生成！单卡也能带的动14B模型", efficient
// inference operators paragraph: the sparse attention computes with Q/K in INT8 and V in
// FP8. Readings: one fp32 scale per (batch, head, block) over all of d, taken over the
// block's valid tokens only; Q over block_q tokens, K and V over block_k tokens.
//   INT8: a = max|x|, s = a/127 and inv = 127/a (IEEE fp32 divisions; both 0 if a = 0),
//         q = clamp(rint(x*inv), -127, 127), rint rounding ties to even.
//   FP8 : (V, and Q and K in the all-FP8 mode, written where the INT8 codes would be)
//         OCP E4M3FN with a power-of-two block scale s = 2^e, e the smallest integer with
//         a <= 448 * 2^e (clamped to [-127, 127], 0 if a = 0), v = e4m3(clamp(x * 2^-e, +-448)),
//         RNE. The attention kernel hands e to the FP8 MFMA as its E8M0 operand scale.
// BF16 mode: K and V are only re-laid out (no rounding).
//
// Output layouts (the attention kernels copy a 64-key sub-tile to LDS as one linear block):
//   Q^  int8  [bh][nQ][bq][128] row-major, pad rows 0.
//   K^  int8  [bh][nK][bk/64][64][128]; the 16-byte chunk c of row r sits at c ^ ((r >> 1) & 7),
//             so 16 lanes reading one chunk of 16 rows hit distinct LDS bank groups.
//   V^T fp8   [bh][nK][bk/64][128][64]; row d lists the 64 keys in the order the attention
//             kernel holds P in registers (key 32kb+8w+4g+r at 32g+16kb+4w+r, so chunk c = 2g+kb
//             of a row holds keys 32kb+8w+4g+r, w,r = 0..3), chunk c of row d at c ^ ((d >> 2) & 3).
//   bf16 mode: K [..][64][128] bf16 with chunk c of row r at c ^ (r & 15); V^T [..][128][64] bf16
//             with key 32kb+8w+4g+r at 16(2kb+w/2)+8g+4(w%2)+r and chunk c of row d at
//             c ^ ((d >> 1) & 7).
//
// Optional prologue of Q and K (PRO), applied before the block means and the quantization in
// the same pass - page "600倍加速，720p视频实时生成！单卡也能带的动14B模型", efficient inference
// operators paragraph, and page "Run Wan2.2-A14B on One RTX 5090: 720p Video in 3.8s", section 4
// (3-D RoPE and RMSNorm as fused kernels). Readings, from the published definitions: RMSNorm
// (Zhang and Sennrich) over the d channels of each head's row with a gain per head and channel,
// y = x / sqrt(mean(x^2) + eps) * g; then the RoFormer rotation (Su et al.) of adjacent channel
// pairs, the 64 pairs split 22/21/21 over the grid axes (t, y, x) of the token, pair j of an
// n-pair group turning by pos * theta^(-j/n). cos and sin come from a table rounded to fp32
// (rope_table_kernel); norm and rotation run as fp32 operations (the values the means and the
// quantizer then see, and the precision the quantizer decides in).
//
// HBM-bound: each input element is read once (16-byte streaming loads) and written once.
#include "sa_internal.h"

namespace sa {

__device__ __forceinline__ void unpack_bf16x8(const uint4& w, float f[8]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = __uint_as_float(u[e] << 16);
    f[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
  }
}

// Position of key rr (0..63 of a sub-tile) in a V^T row, bf16 layout.
__device__ __forceinline__ int vpos_bf16(int rr) {
  const int kb = rr >> 5, q = rr & 31;
  const int g = (q >> 2) & 1, w = q >> 3, r = q & 3;
  return 16 * (2 * kb + (w >> 1)) + 8 * g + 4 * (w & 1) + r;
}

// Max |x| over the block held by the 256 threads of the workgroup.
__device__ __forceinline__ float block_amax(float m, float* red) {
  m = wave_max_f32(m);
  const int t = threadIdx.x;
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  return m;
}

// Pairs of the rotary embedding per grid axis for d = 128: 64 pairs, 22 / 21 / 21 (t, y, x).
constexpr int kPairsT = 22, kPairsY = 21, kPairsX = 21;
static_assert(kPairsT + kPairsY + kPairsX == kD / 2, "every channel pair belongs to one axis");

// cos and sin of every (axis coordinate, pair) angle, in fp64, rounded to fp32. Layout: T rows
// of kPairsT entries (frame axis), then Hg rows of kPairsY, then Wg rows of kPairsX.
__global__ __launch_bounds__(256) void rope_table_kernel(int64_t T, int64_t Hg, int64_t Wg, double theta,
                                                         float2* __restrict__ table) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nt = T * kPairsT, ny = Hg * kPairsY, nx = Wg * kPairsX;
  if (i >= nt + ny + nx) return;
  int64_t pos, j;
  int n;
  if (i < nt) { pos = i / kPairsT; j = i % kPairsT; n = kPairsT; }
  else if (i < nt + ny) { pos = (i - nt) / kPairsY; j = (i - nt) % kPairsY; n = kPairsY; }
  else { pos = (i - nt - ny) / kPairsX; j = (i - nt - ny) % kPairsX; n = kPairsX; }
  const double ang = (double)pos * pow(theta, -(double)j / (double)n);
  table[i] = make_float2((float)cos(ang), (float)sin(ang));
}

// Where this thread's 4 rotary pairs (4*cg ..) sit in the table: axis a (0 = t, 1 = y, 2 = x)
// and the entry offset within the axis section, so that entry = off + coord_a * stride_a.
struct PairSlots {
  int axis[4];
  int32_t off[4];
};
__device__ __forceinline__ PairSlots pair_slots(const QkPrologue& pro, int cg) {
  PairSlots ps;
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    const int p = 4 * cg + pp;
    if (p < kPairsT) { ps.axis[pp] = 0; ps.off[pp] = p; }
    else if (p < kPairsT + kPairsY) { ps.axis[pp] = 1; ps.off[pp] = (int32_t)(pro.grid_t * kPairsT) + (p - kPairsT); }
    else {
      ps.axis[pp] = 2;
      ps.off[pp] = (int32_t)(pro.grid_t * kPairsT + pro.grid_h * kPairsY) + (p - kPairsT - kPairsY);
    }
  }
  return ps;
}

// Lane moves within each 16-lane DPP row, on the vector ALU (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint64_t lo = dpp_u32<CTRL>((uint32_t)u), hi = dpp_u32<CTRL>((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, lo | (hi << 32));
}
// Lane k of each 16-lane row, to the whole row (row_newbcast).
__device__ __forceinline__ float row_lane(float x, int k) {
  const uint32_t u = __float_as_uint(x);
  uint32_t r;
  switch (k) {
    case 0: r = dpp_u32<0x150>(u); break;
    case 1: r = dpp_u32<0x151>(u); break;
    case 2: r = dpp_u32<0x152>(u); break;
    case 3: r = dpp_u32<0x153>(u); break;
    case 4: r = dpp_u32<0x154>(u); break;
    case 5: r = dpp_u32<0x155>(u); break;
    case 6: r = dpp_u32<0x156>(u); break;
    default: r = dpp_u32<0x157>(u); break;
  }
  return __uint_as_float(r);
}

// Exact sum of squares of a row (fp64, of bf16 inputs, so in any order), reduced over the row's
// 16 lanes (lanes 16k .. 16k + 15 hold its 128 channels).
__device__ __forceinline__ double row_sumsq(const float f[8]) {
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += (double)f[e] * (double)f[e];
  // xor-butterfly 8, 4, 2, 1: row_ror 8 is lane i^8; row_ror 4 reaches lane i^4 or i^12, whose
  // partial sums are equal after the first step; the quad permutations are i^2 and i^1
  ss += dpp_f64<0x128>(ss);
  ss += dpp_f64<0x124>(ss);
  ss += dpp_f64<0x4E>(ss);
  ss += dpp_f64<0xB1>(ss);
  return ss;
}

// RMSNorm scaling and 3-D RoPE of one thread's 8 channels (cg*8 ..) of row n, in fp32 operations,
// given the row's r = 1 / sqrt(fp32(ss / d) + eps). Every step is one rounded fp32 operation,
// with no fused multiply-add: y = (x * r) * g, then each product of the rotation and their sum,
// so the result is a function of the IEEE operations only.
__device__ __forceinline__ void rotate_row(float f[8], const float (&g)[8], float rn, const QkPrologue& pro,
                                           const PairSlots& ps, uint32_t n) {
#pragma clang fp contract(off)
  // grid coordinates of token n (row-major t, y, x)
  const uint32_t tt = div_magic(n, pro.hw), rem = n - tt * pro.hw.d;
  const uint32_t yy = div_magic(rem, pro.w), xx = rem - yy * pro.w.d;
  const int32_t coord_off[3] = {(int32_t)tt * kPairsT, (int32_t)yy * kPairsY, (int32_t)xx * kPairsX};
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    const int a = ps.axis[pp];
    const int32_t c_off = a == 0 ? coord_off[0] : (a == 1 ? coord_off[1] : coord_off[2]);
    const float2 cs = pro.table[ps.off[pp] + c_off];
    const float y0 = (f[2 * pp] * rn) * g[2 * pp], y1 = (f[2 * pp + 1] * rn) * g[2 * pp + 1];
    f[2 * pp] = y0 * cs.x - y1 * cs.y;
    f[2 * pp + 1] = y0 * cs.y + y1 * cs.x;
  }
}

// One workgroup (256 threads) per block of one tensor. Work items, per (batch, head): Q
// blocks, then K blocks, then V blocks. Thread t covers columns 8*(t%16).. of rows t/16 + 16k.
// VROWS = block_k: the LDS buffer holds one bf16 V block (VROWS x 128), which also fits the
// 16 x 128 fp64 partial sums of the block means, so block_k = 64 needs only 16 KB and more
// workgroups (bytes in flight) fit on a CU.
// The prologue on one thread's rows (columns 8 cg.. of rows r0 + 16 k2, k2 < nrep, the first at
// token n0 = row0 + r0): RMSNorm then the 3-D rotation, every step a rounded fp32 operation.
// gp: the gains of the thread's 8 columns. Rows at or past L (padding) come out 0.
__device__ __forceinline__ void prologue_rows(const uint4 raw[8], int nrep, const float* gp, const QkPrologue& pro,
                                              int cg, int64_t n0, int64_t L, float xf[8][8]) {
  float g[8];
  const float4 g0 = *(const float4*)gp, g1 = *(const float4*)(gp + 4);
  g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w; g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
  const PairSlots ps = pair_slots(pro, cg);
  // every row's sum of squares; then one correctly rounded 1/sqrt per lane (lane cg takes row
  // cg % 8 of its 16-lane group) handed to the other lanes, instead of 16 equal copies
  double ss[8];
#pragma unroll
  for (int k2 = 0; k2 < 8; ++k2) {
    if (k2 >= nrep) break;  // uniform over the workgroup
    unpack_bf16x8(raw[k2], xf[k2]);
    ss[k2] = row_sumsq(xf[k2]);
  }
  double mine = ss[0];
#pragma unroll
  for (int k2 = 1; k2 < 8; ++k2)
    if (k2 < nrep && (cg & 7) == k2) mine = ss[k2];
  const float rn_mine = 1.0f / sqrtf((float)(mine / (double)kD) + pro.eps);
#pragma unroll
  for (int k2 = 0; k2 < 8; ++k2) {
    if (k2 >= nrep) break;
    const float rn = row_lane(rn_mine, k2);
    // a pad row takes the last token's angles, so the table index stays in range, and is
    // zeroed afterwards (the rotation can turn its zeros into -0, a distinct code)
    const int64_t n = n0 + 16 * k2;
    rotate_row(xf[k2], g, rn, pro, ps, (uint32_t)(n < L ? n : L - 1));
    if (n >= L) {
#pragma unroll
      for (int e = 0; e < 8; ++e) xf[k2][e] = 0.f;
    }
  }
}

// The workgroup id split: per (batch, head), nQ query-block items, then nK key-block and nK
// value-block items.
struct QuantGrid {
  uint32_t nQ, nK;
  DivMagic per_bh, H;
};

template <bool QK_FP8, int VROWS, bool PRO>
__global__ __launch_bounds__(256) void quant_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v, int64_t L,
    int64_t qsb, int64_t qsh, int64_t qsl, int64_t ksb, int64_t ksh, int64_t ksl,
    int64_t vsb, int64_t vsh, int64_t vsl, int bq, int bk, int64_t nQ, int64_t nK,
    int8_t* __restrict__ Qh, int8_t* __restrict__ Kh, uint8_t* __restrict__ Vt,
    float* __restrict__ sq, float* __restrict__ sk, float* __restrict__ sv, double* __restrict__ qmeans,
    double* __restrict__ kmeans, QkPrologue pro, QuantGrid qg) {
  __shared__ float red[4];
  // bf16 block (V), or the fp64 partial column sums of the block means (Q, K)
  __shared__ __attribute__((aligned(16))) uint8_t vtile[VROWS * kD * 2];
  static_assert(VROWS * kD * 2 >= 16 * kD * 8, "the partial sums must fit");
  const int t = threadIdx.x, cg = t & 15, r0 = t >> 4;
  // (batch, head)-major: the nQ + 2 nK items of one head are adjacent, so the workgroups
  // resident at any time mix Q, K and V blocks (measured faster than all Q blocks first, then
  // all K blocks, then all V blocks)
  const uint32_t w = blockIdx.x, bh32 = div_magic(w, qg.per_bh);
  uint32_t blk32 = w - bh32 * qg.per_bh.d;
  int kind;  // 0 = Q, 1 = K, 2 = V
  if (blk32 < qg.nQ) kind = 0;
  else if ((blk32 -= qg.nQ) < qg.nK) kind = 1;
  else { kind = 2; blk32 -= qg.nK; }
  const uint32_t b32 = div_magic(bh32, qg.H);
  const int64_t bh = bh32, blk = blk32, b = b32, h = bh32 - b32 * qg.H.d;
  const int rows = kind == 0 ? bq : bk;
  const int64_t row0 = blk * rows;
  const int count = (int)((L - row0) < rows ? (L - row0) : rows);
  const uint16_t* src;
  int64_t sl;
  if (kind == 0) { src = (const uint16_t*)q + b * qsb + h * qsh; sl = qsl; }
  else if (kind == 1) { src = (const uint16_t*)k + b * ksb + h * ksh; sl = ksl; }
  else { src = (const uint16_t*)v + b * vsb + h * vsh; sl = vsl; }
  src += row0 * sl + cg * 8;

  const int nrep = rows / 16;  // 4 or 8
  uint4 raw[8];
  float amax = 0.f;
#pragma unroll
  for (int k2 = 0; k2 < 8; ++k2) {
    const int r = r0 + 16 * k2;
    raw[k2] = make_uint4(0, 0, 0, 0);
    if (k2 < nrep && r < count) raw[k2] = load_stream(src + (int64_t)r * sl);
  }
  // With the prologue, Q and K rows are normalized and rotated here (pad rows too: they stay 0,
  // since eps > 0); xf then holds the values every later step sees.
  float xf[PRO ? 8 : 1][8];
  const bool pro_rows = PRO && kind < 2;
  if constexpr (PRO) {
    if (pro_rows)
      prologue_rows(raw, nrep, (kind == 0 ? pro.q_gain : pro.k_gain) + h * kD + cg * 8, pro, cg,
                    row0 + r0, L, xf);
  }
  // the values of row k2 of this thread
  auto row_vals = [&](int k2, float f[8]) {
    if constexpr (PRO) {
      if (pro_rows) {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = xf[k2][e];
        return;
      }
    }
    unpack_bf16x8(raw[k2], f);
  };
#pragma unroll
  for (int k2 = 0; k2 < 8; ++k2) {
    if (k2 >= nrep) break;  // rows past the block (xf is only filled up to nrep)
    float f[8];
    row_vals(k2, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(f[e]));
  }
  // Block means for the plan, when asked for (Q and K only): the same fp64 sums in the same
  // order as the pooling kernel (each thread over its rows r0 + 16k in k order, then over the
  // 16 row groups), so the means are bit-identical to those of a separate pooling pass.
  double* means = kind == 0 ? qmeans : (kind == 1 ? kmeans : nullptr);
  if (means) {
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll
    for (int k2 = 0; k2 < 8; ++k2) {
      if (k2 >= nrep) break;
      float f[8];
      row_vals(k2, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += (double)f[e];
    }
    double* part = (double*)vtile;  // [16][kD]
#pragma unroll
    for (int e = 0; e < 8; ++e) part[r0 * kD + cg * 8 + e] = acc[e];
  }
  const float a = block_amax(amax, red);  // (its barrier also publishes the partial sums)
  if (means && t < kD) {
    const double* part = (const double*)vtile;
    double sum = 0.0;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += part[r * kD + t];
    means[(bh * (kind == 0 ? nQ : nK) + blk) * kD + t] = sum / (double)count;
  }
  float s, inv;
  if (kind < 2 && !QK_FP8) {
    s = a > 0.f ? a / 127.0f : 0.f;    // IEEE division
    inv = a > 0.f ? 127.0f / a : 0.f;  // IEEE division
  } else {
    // Power-of-two scale 2^e, e the smallest integer with a <= 448 * 2^e: with a = f * 2^k,
    // f in [0.5, 1), and 448 = 0.875 * 2^9, e = k - 9 if f <= 0.875 else k - 8; clamped to
    // the E8M0 range [-127, 127], and 0 for an all-zero block.
    int k2;
    const float f = frexpf(a, &k2);
    int e = f <= 0.875f ? k2 - 9 : k2 - 8;
    e = a > 0.f ? min(max(e, -127), 127) : 0;
    s = ldexpf(1.f, e);
    inv = ldexpf(1.f, -e);
  }
  if (t == 0) {
    if (kind == 0) sq[bh * nQ + blk] = s;
    else if (kind == 1) sk[bh * nK + blk] = s;
    else sv[bh * nK + blk] = s;
  }
  if (kind < 2) {
#pragma unroll
    for (int k2 = 0; k2 < 8; ++k2) {
      if (k2 >= nrep) break;
      const int r = r0 + 16 * k2;
      float f[8];
      row_vals(k2, f);  // pad rows are 0
      uint32_t packed[2] = {0u, 0u};
      if (QK_FP8) {  // E4M3 codes in the INT8 byte positions
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = fminf(fmaxf(f[4 * h2 + e] * inv, -448.f), 448.f);
          const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
          packed[h2] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float y = rintf(f[e] * inv);
          y = fminf(fmaxf(y, -127.f), 127.f);
          packed[e >> 2] |= ((uint32_t)(int32_t)y & 0xffu) << (8 * (e & 3));
        }
      }
      int8_t* dst;
      if (kind == 0) {
        dst = Qh + ((bh * nQ + blk) * (int64_t)bq + r) * kD + cg * 8;
      } else {
        const int sub = r >> 6, rr = r & 63;
        dst = Kh + (((bh * nK + blk) * (bk >> 6) + sub) * 64 + rr) * kD +
              (((cg >> 1) ^ k_swz(rr)) << 4) + ((cg & 1) << 3);
      }
      *(uint2*)dst = make_uint2(packed[0], packed[1]);
    }
    return;
  }
  // V: FP8, transposed through LDS. The bf16 block goes to LDS row-major (16-byte writes, no
  // bank conflicts); then thread t takes 4 columns d = 4*(t%32).. and one 16-key chunk c of
  // the output row order, reads those 16 keys with 8-byte reads, and writes 4 finished
  // 16-byte chunks (rows d..d+3) of V^T.
#pragma unroll
  for (int k2 = 0; k2 < 8; ++k2) {
    if (k2 >= nrep) break;
    const int r = r0 + 16 * k2;
    *(uint4*)(vtile + (r * kD + cg * 8) * 2) = raw[k2];
  }
  __syncthreads();
  const int dg = t & 31, c = (t >> 5) & 3, sub = t >> 7;
  if (sub < (rows >> 6)) {
    const int g = c >> 1, kb = c & 1;
    uint32_t words[4][4];  // [d][4 keys]
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float f[4][4];  // [key r][d]
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 64 * sub + 32 * kb + 8 * w + 4 * g + r;
        const uint2 x = *(const uint2*)(vtile + (key * kD + 4 * dg) * 2);
        f[r][0] = __uint_as_float(x.x << 16);
        f[r][1] = __uint_as_float(x.x & 0xffff0000u);
        f[r][2] = __uint_as_float(x.y << 16);
        f[r][3] = __uint_as_float(x.y & 0xffff0000u);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float y0 = fminf(fmaxf(f[0][e] * inv, -448.f), 448.f);
        const float y1 = fminf(fmaxf(f[1][e] * inv, -448.f), 448.f);
        const float y2 = fminf(fmaxf(f[2][e] * inv, -448.f), 448.f);
        const float y3 = fminf(fmaxf(f[3][e] * inv, -448.f), 448.f);
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
        words[e][w] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, lo, true);
      }
    }
    uint8_t* dst = Vt + ((bh * nK + blk) * (int64_t)(bk >> 6) + sub) * (64 * kD);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d = 4 * dg + e;
      *(uint4*)(dst + d * 64 + ((c ^ v_swz(d)) << 4)) =
          make_uint4(words[e][0], words[e][1], words[e][2], words[e][3]);
    }
  }
}

// bf16 mode: K (WITH_K) and V of each key block into the attention kernel's tile layout.
// Without the prologue (WITH_K) the pass also records that the attention reads the caller's Q
// (q_flag = 0); with it, K comes from prologue_bf16_kernel, which sets q_flag = 1.
template <bool WITH_K>
__global__ __launch_bounds__(256) void layout_bf16_kernel(
    const void* __restrict__ k, const void* __restrict__ v, DivMagic H, int64_t L, int64_t ksb,
    int64_t ksh, int64_t ksl, int64_t vsb, int64_t vsh, int64_t vsl, int bk, DivMagic nKd,
    uint16_t* __restrict__ Kt, uint16_t* __restrict__ Vt, int32_t* __restrict__ q_flag) {
  if (WITH_K && blockIdx.x == 0 && threadIdx.x == 0) *q_flag = 0;
  __shared__ __attribute__((aligned(16))) uint16_t vtile[128 * 64];  // one 64-key sub-tile
  const int t = threadIdx.x, cg = t & 15, r0 = t >> 4;
  const uint32_t w = blockIdx.x, bh32 = div_magic(w, nKd), b32 = div_magic(bh32, H);
  const int64_t nK = nKd.d, bh = bh32, blk = w - bh32 * nKd.d, b = b32, h = bh32 - b32 * H.d;
  const int64_t row0 = blk * bk;
  const int count = (int)((L - row0) < bk ? (L - row0) : bk);
  const uint16_t* ks = (const uint16_t*)k + b * ksb + h * ksh + row0 * ksl + cg * 8;
  const uint16_t* vs = (const uint16_t*)v + b * vsb + h * vsh + row0 * vsl + cg * 8;
  for (int sub = 0; sub < bk / 64; ++sub) {
    uint16_t* kdst = Kt + ((bh * nK + blk) * (bk >> 6) + sub) * 64 * kD;
    uint16_t* vdst = Vt + ((bh * nK + blk) * (bk >> 6) + sub) * 64 * kD;
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      const int rr = r0 + 16 * k2, r = sub * 64 + rr;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (r < count) {
        if (WITH_K) kv = *(const uint4*)(ks + (int64_t)r * ksl);
        vv = *(const uint4*)(vs + (int64_t)r * vsl);
      }
      if (WITH_K) *(uint4*)(kdst + rr * kD + ((cg ^ bk_swz(rr)) << 3)) = kv;
      const int pos = vpos_bf16(rr);
      const uint16_t vals[8] = {(uint16_t)(vv.x & 0xffff), (uint16_t)(vv.x >> 16),
                                (uint16_t)(vv.y & 0xffff), (uint16_t)(vv.y >> 16),
                                (uint16_t)(vv.z & 0xffff), (uint16_t)(vv.z >> 16),
                                (uint16_t)(vv.w & 0xffff), (uint16_t)(vv.w >> 16)};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = cg * 8 + e;
        vtile[d * 64 + (((pos >> 3) ^ bv_swz(d)) << 3) + (pos & 7)] = vals[e];
      }
    }
    __syncthreads();
    for (int o = t * 8; o < 64 * kD; o += 256 * 8) *(uint4*)(vdst + o) = *(const uint4*)(vtile + o);
    __syncthreads();
  }
}

// bf16 mode with the prologue: one workgroup per Q or K block (per (batch, head): nQ Q blocks,
// then nK K blocks). The rows are normalized and rotated with quant_kernel's fp32 operations,
// their fp64 block means taken in the same order (so they equal those of the quantized modes),
// and the values rounded to bf16 (RNE) for the bf16 MFMAs: Q row-major into the workspace's Q
// region [bh][nQ][bq][128] (pad rows 0), K into the bf16 tile layout. Thread t covers columns
// 8*(t%16).. of rows t/16 + 16k.
__global__ __launch_bounds__(256) void prologue_bf16_kernel(
    const void* __restrict__ q, const void* __restrict__ k, int64_t L, int64_t qsb, int64_t qsh, int64_t qsl,
    int64_t ksb, int64_t ksh, int64_t ksl, int bq, int bk, QuantGrid qg, uint16_t* __restrict__ Qw,
    uint16_t* __restrict__ Kt, double* __restrict__ qmeans, double* __restrict__ kmeans,
    int32_t* __restrict__ q_flag, QkPrologue pro) {
  __shared__ __attribute__((aligned(16))) double part[16 * kD];
  const int t = threadIdx.x, cg = t & 15, r0 = t >> 4;
  const uint32_t w = blockIdx.x, bh32 = div_magic(w, qg.per_bh);
  uint32_t blk32 = w - bh32 * qg.per_bh.d;
  const int kind = blk32 < qg.nQ ? 0 : 1;  // 0 = Q, 1 = K
  if (kind) blk32 -= qg.nQ;
  const uint32_t b32 = div_magic(bh32, qg.H);
  const int64_t bh = bh32, blk = blk32, b = b32, h = bh32 - b32 * qg.H.d;
  const int rows = kind == 0 ? bq : bk;
  const int64_t row0 = blk * rows;
  const int count = (int)((L - row0) < rows ? (L - row0) : rows);
  const int64_t sl = kind == 0 ? qsl : ksl;
  const uint16_t* src = (kind == 0 ? (const uint16_t*)q + b * qsb + h * qsh : (const uint16_t*)k + b * ksb + h * ksh) +
                        row0 * sl + cg * 8;
  if (w == 0 && t == 0) *q_flag = 1;
  const int nrep = rows / 16;  // 4 or 8
  uint4 raw[8];
#pragma unroll
  for (int k2 = 0; k2 < 8; ++k2) {
    const int r = r0 + 16 * k2;
    raw[k2] = make_uint4(0, 0, 0, 0);
    if (k2 < nrep && r < count) raw[k2] = load_stream(src + (int64_t)r * sl);
  }
  float xf[8][8];
  prologue_rows(raw, nrep, (kind == 0 ? pro.q_gain : pro.k_gain) + h * kD + cg * 8, pro, cg, row0 + r0, L, xf);
  // block means: the order of quant_kernel (rows r0 + 16 k in k order, then the 16 row groups)
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll
  for (int k2 = 0; k2 < 8; ++k2) {
    if (k2 >= nrep) break;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += (double)xf[k2][e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[r0 * kD + cg * 8 + e] = acc[e];
  __syncthreads();
  if (t < kD) {
    double sum = 0.0;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += part[r * kD + t];
    (kind == 0 ? qmeans : kmeans)[(bh * (kind == 0 ? qg.nQ : qg.nK) + blk) * kD + t] = sum / (double)count;
  }
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int k2 = 0; k2 < 8; ++k2) {
    if (k2 >= nrep) break;
    const int r = r0 + 16 * k2;
    uint32_t wd[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f2 pv = {xf[k2][2 * e], xf[k2][2 * e + 1]};
      wd[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pv, bf2));  // RNE
    }
    uint16_t* dst;
    if (kind == 0) {
      dst = Qw + ((bh * qg.nQ + blk) * (int64_t)bq + r) * kD + cg * 8;
    } else {
      const int sub = r >> 6, rr = r & 63;
      dst = Kt + (((bh * qg.nK + blk) * (bk >> 6) + sub) * 64 + rr) * kD + ((cg ^ bk_swz(rr)) << 3);
    }
    *(uint4*)dst = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  }
}

void launch_quant(const TensorView& q, const TensorView& k, const TensorView& v, int64_t B,
                  int64_t H, int64_t L, int bq, int bk, const sa_forward_layout& lay, char* ws,
                  double* qmeans, double* kmeans, bool qk_fp8, const QkPrologue* pro, hipStream_t s) {
  const int64_t BH = B * H;
  const dim3 grid((unsigned)(BH * (lay.nQ + 2 * lay.nK)));
  // every id stays below 2^24 (the entry points bound B*H*(nQ + 2 nK) by 2^32 / 256)
  const QuantGrid qg{(uint32_t)lay.nQ, (uint32_t)lay.nK, div_magic_for((uint32_t)(lay.nQ + 2 * lay.nK)),
                     div_magic_for((uint32_t)H)};
  QkPrologue p{};
  if (pro) {
    p = *pro;
    // token n < 2^31 to grid coordinates: n / (grid_h * grid_w), then the rest / grid_w
    p.hw = div_magic_for((uint32_t)(p.grid_h * p.grid_w));
    p.w = div_magic_for((uint32_t)p.grid_w);
    const int64_t entries = p.grid_t * kPairsT + p.grid_h * kPairsY + p.grid_w * kPairsX;
    rope_table_kernel<<<dim3((unsigned)((entries + 255) / 256)), 256, 0, s>>>(p.grid_t, p.grid_h, p.grid_w,
                                                                                p.theta, p.table);
  }
#define SA_QUANT(F8, VR, PR) quant_kernel<F8, VR, PR>
  auto kern = pro ? (bk == 64 ? (qk_fp8 ? SA_QUANT(true, 64, true) : SA_QUANT(false, 64, true))
                              : (qk_fp8 ? SA_QUANT(true, 128, true) : SA_QUANT(false, 128, true)))
                  : (bk == 64 ? (qk_fp8 ? SA_QUANT(true, 64, false) : SA_QUANT(false, 64, false))
                              : (qk_fp8 ? SA_QUANT(true, 128, false) : SA_QUANT(false, 128, false)));
#undef SA_QUANT
  kern<<<grid, 256, 0, s>>>(q.data, k.data, v.data, L, q.sb, q.sh, q.sl, k.sb, k.sh, k.sl, v.sb,
                            v.sh, v.sl, bq, bk, lay.nQ, lay.nK, (int8_t*)(ws + lay.q_off),
                            (int8_t*)(ws + lay.k_off), (uint8_t*)(ws + lay.v_off),
                            (float*)(ws + lay.sq_off), (float*)(ws + lay.sk_off),
                            (float*)(ws + lay.sv_off), qmeans, kmeans, p, qg);
}

size_t rope_table_bytes(int64_t T, int64_t Hg, int64_t Wg) {
  return (size_t)(T * kPairsT + Hg * kPairsY + Wg * kPairsX) * sizeof(float2);
}

void launch_layout_bf16(const TensorView& k, const TensorView& v, int64_t B, int64_t H, int64_t L,
                        int bk, const sa_forward_layout& lay, char* ws, hipStream_t s) {
  const dim3 grid((unsigned)(B * H * lay.nK));
  layout_bf16_kernel<true><<<grid, 256, 0, s>>>(k.data, v.data, div_magic_for((uint32_t)H), L, k.sb, k.sh, k.sl,
                                                v.sb, v.sh, v.sl, bk, div_magic_for((uint32_t)lay.nK),
                                                (uint16_t*)(ws + lay.k_off), (uint16_t*)(ws + lay.v_off),
                                                (int32_t*)(ws + lay.sq_off));
}

void launch_prologue_bf16(const TensorView& q, const TensorView& k, const TensorView& v, int64_t B, int64_t H,
                          int64_t L, int bq, int bk, const sa_forward_layout& lay, char* ws, double* qmeans,
                          double* kmeans, const QkPrologue& pro, hipStream_t s) {
  const int64_t BH = B * H;
  QkPrologue p = pro;
  p.hw = div_magic_for((uint32_t)(p.grid_h * p.grid_w));
  p.w = div_magic_for((uint32_t)p.grid_w);
  const int64_t entries = p.grid_t * kPairsT + p.grid_h * kPairsY + p.grid_w * kPairsX;
  rope_table_kernel<<<dim3((unsigned)((entries + 255) / 256)), 256, 0, s>>>(p.grid_t, p.grid_h, p.grid_w, p.theta,
                                                                              p.table);
  // every id stays below 2^24 (the entry points bound B*H*(nQ + 2 nK) by 2^32 / 256)
  const QuantGrid qg{(uint32_t)lay.nQ, (uint32_t)lay.nK, div_magic_for((uint32_t)(lay.nQ + lay.nK)),
                     div_magic_for((uint32_t)H)};
  prologue_bf16_kernel<<<dim3((unsigned)(BH * (lay.nQ + lay.nK))), 256, 0, s>>>(
      q.data, k.data, L, q.sb, q.sh, q.sl, k.sb, k.sh, k.sl, bq, bk, qg, (uint16_t*)(ws + lay.q_off),
      (uint16_t*)(ws + lay.k_off), qmeans, kmeans, (int32_t*)(ws + lay.sq_off), p);
  layout_bf16_kernel<false><<<dim3((unsigned)(BH * lay.nK)), 256, 0, s>>>(
      k.data, v.data, div_magic_for((uint32_t)H), L, k.sb, k.sh, k.sl, v.sb, v.sh, v.sl, bk,
      div_magic_for((uint32_t)lay.nK), (uint16_t*)(ws + lay.k_off), (uint16_t*)(ws + lay.v_off),
      (int32_t*)(ws + lay.sq_off));
}

}  // namespace sa
