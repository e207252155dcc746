// Block-sparse attention over the kept tiles.
//
// Page "600倍加速，720p视频实时生成！单卡也能带的动14B模型", dynamic sparse quantized
// attention paragraph: only the activated tiles are computed and they are computed densely;
// efficient inference operators paragraph: Q/K in INT8 and V in FP8. Page "Run Wan2.2-A14B
// on One RTX 5090", section 3: dense computation inside the surviving blocks. Readings: no
// causal mask; softmax scale 1/sqrt(d); tiles visited in ascending key-block order; online
// softmax in fp32 in the log2 domain; P scaled by 2^8 and rounded to FP8 E4M3 (RNE) for the
// PV product, the row sum taken over those rounded weights (the ones V is multiplied by).
//
// Work split: one workgroup per (batch, head, query block), block_q/32 wavefronts of 32
// query rows each. All wavefronts of a workgroup share the block's kept key list, so every
// kept 64-key sub-tile (K^ 8 KB + V^T 8 KB in INT8/FP8 mode) is copied once into LDS (a
// three-slot ring; in bf16 mode K in two slots and V^T in one) and read by all of them.
//
// Per wavefront and 64-key sub-tile, INT8/FP8 mode:
//   S^T[64 keys][32 queries] = K^ Q^^T : 8 x v_mfma_i32_32x32x32_i8, exact int32.
//     The transposed product leaves each lane with one query row (lane % 32) and 32 of its
//     64 keys (the other 32 in lane ^ 32), so row max and row sum are lane-local but for a
//     single exchange with the partner lane.
//   x = S * g with g = fl(fl(s_q s_k) * fl(sm log2 e)); reference max m' = the running max
//   rounded up to an integer; p256 = 2^(x - (m' - 8)) = p * 2^8;
//   P^ = fp8(p256) packed straight from the accumulator registers into the B operand of
//   O^T[128 d][32 q] += V^T P^^T : 4 x v_mfma_f32_32x32x64_f8f6f4 (V^T's key order in memory
//   matches the register order of P, so no shuffle is needed).
//   The per-block V scale 2^e_v and the tile's factor 2^(m' - m0) (m0 a per-row base) are
//   E8M0 operand scales the MFMA applies, so the accumulators are not rescaled between
//   tiles; l += sum of P^ (one more MFMA, row_sum_fp8) times the tile's factor; the output
//   is acc / l.
#include <type_traits>

#include "sa_internal.h"

namespace sa {

// Score bias. The QK^T accumulators start from the bit pattern of 1.5f (0x3FC00000) in every
// element. Its mantissa field 2^22 exceeds every |S| <= 128 * 127^2 = 2,064,512, so the int32
// sum bits(1.5f) + S stays in the binade [1, 2): read as a float it is exactly 1.5 + S * 2^-23.
// The exponent x - m' + 8 = S g - m' + 8 is then one fused multiply-add of that float with
// gx = g22 * 2^23, plus the addend (8 - m') - 1.5 gx, and the 32 int-to-float conversions per
// lane and sub-tile are not needed. g22 is g rounded to 22 significant bits (relative change
// below 2^-22), which makes 1.5 gx exact in fp32 and the addend's subtraction of the integer
// 8 - m' exact whenever |8 - m'| <= 1.5 gx / 3 (otherwise off by half an ulp of a value no
// larger than 4 |8 - m'|). Both stay far below the logit error that moves an FP8 code.
constexpr float kBiasF = 1.5f;
constexpr int kBiasBits = 0x3FC00000;
static_assert((1 << 22) > 128 * 127 * 127, "every INT8 score must fit the bias's binade");

// g rounded to 22 significant bits (nearest, ties away: the two dropped bits decide) and
// scaled by 2^23, for the biased scores above.
__device__ __forceinline__ float bias_gx(float g) {
  return __int_as_float((__float_as_int(g) + 2) & ~3) * 8388608.f;
}

// ---------------------------------------------------------------------------------------
// shared pieces
// ---------------------------------------------------------------------------------------

// Linear copy of a sub-tile operand from global memory to LDS through registers:
// thread t moves 16-byte pieces t, t + NT, ... (kPer of them).
template <int kPer, int NT>
__device__ __forceinline__ void tile_load(v4i (&r)[kPer], const uint8_t* __restrict__ src, int t) {
#pragma unroll
  for (int k = 0; k < kPer; ++k) r[k] = *(const v4i*)(src + (k * NT + t) * 16);
}
template <int kPer, int NT>
__device__ __forceinline__ void tile_store(const v4i (&r)[kPer], uint8_t* dst, int t) {
#pragma unroll
  for (int k = 0; k < kPer; ++k) *(v4i*)(dst + (k * NT + t) * 16) = r[k];
}

// S^T of one 64-key INT8 sub-tile for one wavefront: acc[kb] holds keys 32kb..32kb+31.
// ldsK: [64][128] int8 with the chunk swizzle; qB[c] = Q^ bytes 32c+16g..+15 of query n.
// The int32 accumulators start from c_init (zeros for the exact tile; the attention kernel
// passes the score bias, so each result is an fp32 bit pattern that needs no conversion).
// The K^ fragments of the first two k steps are read before the first MFMA and each later
// pair right after the MFMAs that free its registers, so four LDS reads are in flight at the
// start (the scheduling barriers keep the compiler from pairing each read with its MFMA).
__device__ __forceinline__ void qk_subtile_i8(const uint8_t* ldsK, const v4i qB[4], int n, int g,
                                              v16i acc[2], const v16i& c_init) {
  // fragment (kb, c): rows n and n + 32 share the swizzle, so kb = 1 is 32 rows (4096 bytes) on
  const uint8_t* base = ldsK + n * kD;
  const int sw = k_swz(n);
  auto frag = [&](int kb, int c) { return *(const v4i*)(base + 32 * kD * kb + (((2 * c + g) ^ sw) << 4)); };
  v4i x0 = frag(0, 0), x1 = frag(1, 0), y0 = frag(0, 1), y1 = frag(1, 1);
  __builtin_amdgcn_sched_barrier(0);
  v16i c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(x0, qB[0], c_init, 0, 0, 0);
  v16i c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(x1, qB[0], c_init, 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  x0 = frag(0, 2);
  x1 = frag(1, 2);
  __builtin_amdgcn_sched_barrier(0);
  c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(y0, qB[1], c0, 0, 0, 0);
  c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(y1, qB[1], c1, 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  y0 = frag(0, 3);
  y1 = frag(1, 3);
  __builtin_amdgcn_sched_barrier(0);
  c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(x0, qB[2], c0, 0, 0, 0);
  c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(x1, qB[2], c1, 0, 0, 0);
  c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(y0, qB[3], c0, 0, 0, 0);
  c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(y1, qB[3], c1, 0, 0, 0);
  acc[0] = c0;
  acc[1] = c1;
}

// The same S^T with E4M3 Q^ and K^ (all-FP8 mode), in fp32 and already multiplied by the two
// power-of-two block scales (E8M0 codes k_code, q_code, applied by the MFMA). The operands are
// the INT8 path's 16-byte fragments taken in pairs: chunks 2c and 2c+1 form the 32 bytes an
// FP8 32x32x64 MFMA takes per lane, and A and B pair them the same way, so every d is summed
// once.
__device__ __forceinline__ void qk_subtile_f8(const uint8_t* ldsK, const v4i qB[4], int n, int g,
                                              int k_code, int q_code, v16f acc[2]) {
  v4i a[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = 32 * kb + n;
#pragma unroll
    for (int c = 0; c < 4; ++c) a[kb][c] = *(const v4i*)(ldsK + row * kD + (((2 * c + g) ^ k_swz(row)) << 4));
  }
  v16f c0 = {}, c1 = {};
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const v4i b0 = qB[2 * cc], b1 = qB[2 * cc + 1];
    const v8i b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    const v4i x0 = a[0][2 * cc], x1 = a[0][2 * cc + 1], y0 = a[1][2 * cc], y1 = a[1][2 * cc + 1];
    const v8i a0 = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    const v8i a1 = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, b, c0, 0, 0, 0, k_code, 0, q_code);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, b, c1, 0, 0, 0, k_code, 0, q_code);
  }
  acc[0] = c0;
  acc[1] = c1;
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

// Two floats to a bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const f2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2));
}

// Combine a lane's value with that of lane l ^ 32 (the other half of the wavefront) through
// one cross-half swap instead of an LDS permute.
__device__ __forceinline__ int xor32_max(int x) {
  const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ float xor32_maxf(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// Sum of the 64 FP8 weights of a query row in P (its lane's 32 bytes and those of lane ^ 32),
// on the matrix cores: one scaled 16x16x128 FP8 MFMA (unit scales) with a 0/1 operand A. As
// its B operand, P gives lane l's 32 bytes to column l % 16, k group l / 16; A's row i holds
// ones (E4M3 1.0) in the k groups whose lanes carry query (i/4 odd ? 16 : 0) + column, so D row
// 4 (l / 16), read by lane l, is the sum for the lane's own query l % 32 over both key halves.
// The products are exact and the 64-term sums land within 2^-10.9 of their largest term
// (exact when the weights span at most four binades); the VALU is spared 32 additions per
// sub-tile, and the matrix cores spend half the cycles of four 16x16x32 FP8 MFMAs.
__device__ __forceinline__ float row_sum_fp8(const v8i& P) {
  const int lane = __lane_id();
  const int f8 = ((((lane & 15) >> 2) & 1) == ((lane >> 4) & 1)) ? 0x38383838 : 0;
  const v8i ones = {f8, f8, f8, f8, f8, f8, f8, f8};
  const v4f d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, P, (v4f){}, 0, 0, 0, 127, 0, 127);
  return d[0];
}

// ---------------------------------------------------------------------------------------
// INT8 QK^T + FP8 PV
// ---------------------------------------------------------------------------------------
// Per-row softmax state (one query row per lane pair). m: the reference max, an integer in
// the log2 domain (the running max rounded up), so P's FP8 scale is a power of two. The
// accumulators and l are kept in units of 2^(m0 - m) of the true online-softmax state, m0 a
// base reference max: tile j adds its P V^T scaled by 2^(m_j - m0), which the FP8 MFMA applies
// as an E8M0 operand scale, so the accumulators are never multiplied on tile boundaries. The
// output acc / l is the same (the common factor cancels).
struct SoftmaxState {
  float m, m0, l;
};

// Largest tile exponent m_j - m0 let into the accumulators before they are brought back to
// the current reference (an exact power-of-two rescale, needed only when a row's max rises
// by more than this many binades after its first tile).
constexpr float kMaxRel = 64.f;
constexpr float kBase0 = -1.0e30f;  // initial base of a row: the first tile always rebases

// E8M0 code (biased exponent) of a power-of-two block scale: 2^e -> 127 + e. The fp32 bit
// pattern already holds it, also for 2^-127 (a subnormal, exponent field 0 = code 0).
__device__ __forceinline__ int e8m0_code(float pow2) { return (int)(__float_as_uint(pow2) >> 23); }

// Softmax and PV of one 64-key sub-tile for one wavefront, given its S^T accumulators.
// PARTIAL: keys at or past `valid` are padding (only the last key block of a sequence whose
// length is not a multiple of 64 has them). v_code: E8M0 code of the block's V scale.
// SV: v16i (exact INT8 scores, x = S * gt) or v16f (FP8 scores, already scaled, gt = sm log2 e).
template <bool PARTIAL, typename SV>
__device__ __forceinline__ void softmax_pv_i8f8(const SV S[2], const uint8_t* ldsV, int n, int g,
                                                int valid, float gt, int v_code, SoftmaxState& st,
                                                v16f acc[4], uint32_t vlo, uint32_t vhi) {
  constexpr bool kInt = std::is_same<SV, v16i>::value;
  // The softmax's VALU work issues at a raised wave priority, dropped again before the PV
  // MFMAs: with three wavefronts per SIMD the one in its softmax then gets the issue slots
  // first while the others wait on their MFMAs (about 2 % faster at 720p; raising it around
  // the MFMAs instead was much slower).
  __builtin_amdgcn_s_setprio(1);
  float smax;
  if constexpr (kInt) {
    int mx = INT_MIN;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (!PARTIAL || acc_key(kb, v, g) < valid) mx = max(mx, S[kb][v]);
    // The biased scores are positive floats, which order like their bit patterns; the
    // difference from kBiasF is exact (both in one binade), so smax is the integer max S.
    smax = (__int_as_float(xor32_max(mx)) - kBiasF) * 8388608.f;
  } else {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (!PARTIAL || acc_key(kb, v, g) < valid) mx = fmaxf(mx, S[kb][v]);
    smax = xor32_maxf(mx);
  }
  const float m_new = fmaxf(st.m, ceilf(smax * gt));
  // The base starts at kBase0, far below any reference max, so the first tile takes the
  // rescale below (factor 2^-256 = 0 on the still-zero accumulators and row sum; base := m')
  // and no tile needs a test for being the first.
  float m0 = st.m0;
  float rel = m_new - m0;  // a small non-negative integer after the first tile
  if (__ballot(rel > kMaxRel)) {
    const bool far = rel > kMaxRel;
    const float f = far ? __builtin_amdgcn_ldexpf(1.f, (int)fmaxf(-rel, -256.f)) : 1.f;  // exact power of two
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] *= f;
    st.l *= f;
    m0 = far ? m_new : m0;
    rel = far ? 0.f : rel;
  }
  // p * 2^8 = 2^(x - m' + 8). The addend is kept as a plain register operand (no negation
  // modifier): the plain three-VGPR form of v_fma_f32 issues at about twice the rate.
  float gx = gt, nb = 8.f - m_new;
  if constexpr (kInt) {
    // S g22 = F gx - 1.5 gx, F the biased accumulator read as a float (see kBiasF)
    gx = bias_gx(gt);
    nb = nb - kBiasF * gx;
  }
  v8i P;
#pragma unroll
  for (int w4 = 0; w4 < 8; ++w4) {
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kb = w4 >> 2, v = 4 * (w4 & 3) + e;
      const float sv = kInt ? __int_as_float((int)S[kb][v]) : (float)S[kb][v];
      p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, gx, nb));
      if (PARTIAL && acc_key(kb, v, g) >= valid) p[e] = 0.f;
    }
    // The low half is written first and the high half second, so the word's old value does
    // not matter: start from p[0]'s register, which dies here (no register move).
    const int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __float_as_int(p[0]), false);
    P[w4] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wd, true);
  }
  const int irel = (int)rel;
  st.l += __builtin_amdgcn_ldexpf(row_sum_fp8(P), irel);
  const int p_code = 127 + irel;  // P^'s E8M0 scale: 2^(m' - m0)
  __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    // row d = 32 db + n: the db part is a constant offset, the lane part (vlo, vhi) is fixed
    const v4i lo = *(const v4i*)(ldsV + 2048 * db + vlo);
    const v4i hi = *(const v4i*)(ldsV + 2048 * db + vhi);
    const v8i a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    // O^T += (2^e_v V^T) (2^(m' - m0) P^): E8M0 scale codes v_code and p_code.
    acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, P, acc[db], 0, 0, 0, v_code, 0, p_code);
  }
  st.m = m_new;
  st.m0 = m0;
}

// Make sure values loaded from global memory have arrived (the compiler then needs no
// wait on them inside the loop that follows).
template <typename T>
__device__ __forceinline__ void settle(const T& x) {
  asm volatile("" : : "v"(x));
}

// Asynchronous global -> LDS copy of one sub-tile (K^ 8 KB then V^T 8 KB), 16 bytes per lane
// per instruction: lane l of wave w lands at dst + ((k*NT + 64w + l) * 16), the same linear
// image as the source.
template <int NT>
__device__ __forceinline__ void tile_dma(const uint8_t* __restrict__ ksrc, const uint8_t* __restrict__ vsrc,
                                         uint8_t* dst, int t) {
  constexpr int kPer = 64 * kD / (16 * NT);
  const int wbase = t & ~63;
#pragma unroll
  for (int k = 0; k < kPer; ++k)
    __builtin_amdgcn_global_load_lds(
        (const void __attribute__((address_space(1)))*)(ksrc + (k * NT + t) * 16),
        (void __attribute__((address_space(3)))*)(dst + (k * NT + wbase) * 16), 16, 0, 0);
#pragma unroll
  for (int k = 0; k < kPer; ++k)
    __builtin_amdgcn_global_load_lds(
        (const void __attribute__((address_space(1)))*)(vsrc + (k * NT + t) * 16),
        (void __attribute__((address_space(3)))*)(dst + 64 * kD + (k * NT + wbase) * 16), 16, 0, 0);
}

// The same copy issued through inline asm, for the INT8/FP8 kernel's main loop. The compiler's
// wait insertion tracks LDS-DMA copies by destination but loses that information at a loop
// header, and would then wait for every copy in flight (including the one just started two
// sub-tiles ahead) before the first LDS read of each iteration. Copies it cannot see are
// ordered only by the kernel's own vmcnt waits and barriers, which already cover them. The
// compiler loads M0 (the wave's LDS destination) for the asm; the s_nop is the one wait state
// an M0 write needs before an LDS DMA.
//
// The source is addressed as a wave-uniform SGPR base plus a per-lane 32-bit offset and M0 is
// computed from the buffer's LDS address, so a copy costs no VALU instruction.
__device__ __forceinline__ void lds_dma16(const uint8_t* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(size_t)(__attribute__((address_space(3))) const uint8_t*)p;
}

// One sub-tile (K^ then V^T, 8 KB each) from the wave-uniform sources ksrc, vsrc into dst.
// wave_lds = 1024 * wavefront index (the LDS offset of the wavefront's first 16-byte piece).
template <int NT>
__device__ __forceinline__ void tile_dma_asm(const uint8_t* ksrc, const uint8_t* vsrc, uint8_t* dst, int t,
                                             uint32_t wave_lds) {
  constexpr int kPer = 64 * kD / (16 * NT);
  const uint32_t voff = (uint32_t)t * 16u;
  const uint32_t base = lds_addr(dst) + wave_lds;
#pragma unroll
  for (int k = 0; k < kPer; ++k) lds_dma16(ksrc + k * NT * 16, voff, base + k * NT * 16);
#pragma unroll
  for (int k = 0; k < kPer; ++k) lds_dma16(vsrc + k * NT * 16, voff, base + 64 * kD + k * NT * 16);
}

typedef const __attribute__((address_space(4))) int32_t* cint32_p;
typedef const __attribute__((address_space(4))) float* cfloat_p;

// Workgroup barrier for the DMA pipeline. __syncthreads() (and any release fence on LDS)
// makes the compiler wait for every outstanding LDS-DMA copy, including the ones issued a
// sub-tile ahead on purpose. In the loop the only LDS writes are those copies, and each
// wavefront waits for the ones it needs with an explicit vector-memory count before the
// barrier, so the barrier itself needs no release: an acquire on LDS keeps the reads that
// follow from moving above it.
__device__ __forceinline__ void dma_barrier() {
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0xF70); }  // vmcnt(0)

// DMA instructions one thread issues per sub-tile (K^ and V^T, 16 bytes each).
template <int NT>
constexpr int kDmaPerTile = 2 * 64 * kD / (16 * NT);

// Main loop: sub-tile u is computed from one of three LDS buffers while sub-tiles u+1 and u+2
// are being copied by DMA into the other two (two sub-tiles of lead hide gathers that miss
// L2). The loop is unrolled three times so that every step's buffers are constant offsets
// into the ring; the copies are issued through inline asm that the compiler's wait insertion
// does not see, and are ordered only by the kernel's own waits and barriers.
// Three workgroups' worth of wavefronts per SIMD are requested: with fewer resident
// wavefronts the VALU cannot issue at its full rate while another wavefront runs MFMAs.
// F8QK: Q^ and K^ are E4M3 with power-of-two scales (all-FP8 mode) instead of INT8.
template <int BQ, int NSUB, bool F8QK>
__global__ __launch_bounds__(BQ * 2, 3) void attn_i8f8_kernel(
    const int8_t* __restrict__ Qh, const uint8_t* __restrict__ Kh, const uint8_t* __restrict__ Vt,
    const float* __restrict__ sq, const float* __restrict__ sk, const float* __restrict__ sv,
    const int32_t* __restrict__ plan, int64_t H, int L, int64_t nQ, int nK, int n_keep,
    float c_log2, __bf16* __restrict__ out, int64_t ob, int64_t oh, int64_t ol, int64_t total) {
  constexpr int NT = BQ * 2;
  constexpr int kSubBytes = 64 * kD;  // one operand of a sub-tile
  // The waits below put the copy count in the low four bits of s_waitcnt's vmcnt field.
  static_assert(kDmaPerTile<NT> < 16, "vmcnt immediate 0xF70 | n needs n < 16");
  // The three ring buffers are one array, so the LDS reads of every buffer share their lane
  // address registers (the buffer is an immediate offset).
  __shared__ __attribute__((aligned(16))) uint8_t ring[3 * 2 * kSubBytes];
  uint8_t* const buf0 = ring;
  uint8_t* const buf1 = ring + 2 * kSubBytes;
  uint8_t* const buf2 = ring + 4 * kSubBytes;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63, n = lane & 31, g = lane >> 5;
  const uint32_t wave_lds = __builtin_amdgcn_readfirstlane((uint32_t)wave * 1024u);
  const int64_t w = xcd_remap(blockIdx.x, total);
  const int64_t bh = w / nQ, i = w % nQ;
  const int64_t b = bh / H, h = bh % H;
  // Plan entries and block scales are read through the constant address space: uniform
  // addresses there become scalar loads, which the DMA waits (vector-memory counter) ignore.
  const cint32_p prow = (cint32_p)(plan + (bh * nQ + i) * n_keep);
  const cfloat_p skh = (cfloat_p)(sk + bh * nK);
  const cfloat_p svh = (cfloat_p)(sv + bh * nK);
  const uint8_t* Kb = Kh + bh * (int64_t)nK * NSUB * kSubBytes;
  const uint8_t* Vb = Vt + bh * (int64_t)nK * NSUB * kSubBytes;
  const int U = n_keep * NSUB;

  v4i qB[4];
  load_q_i8(Qh + (bh * nQ + i) * (int64_t)BQ * kD, 32 * wave + n, g, qB);
  const float s_q = sq[bh * nQ + i];
  const int q_code = e8m0_code(s_q);  // all-FP8 mode: Q^'s block scale as an E8M0 code
#pragma unroll
  for (int c = 0; c < 4; ++c) settle(qB[c]);

  auto blk = [&](int u) -> int { return prow[(u < U ? u : U - 1) / NSUB]; };
  auto dma = [&](int u, uint8_t* dst) {
    int j = blk(u);
    j = (unsigned)j < (unsigned)nK ? j : 0;
    const int64_t off = ((int64_t)j * NSUB + (u % NSUB)) * kSubBytes;
    tile_dma_asm<NT>(Kb + off, Vb + off, dst, t, wave_lds);
  };
  auto sub_valid = [&](int j, int u) -> int {
    return (unsigned)j < (unsigned)nK ? min(64, L - (j * (64 * NSUB) + 64 * (u % NSUB))) : 0;
  };

  // V^T fragment offsets of this lane inside a sub-tile (row n of each 32-row group, its two
  // 16-byte chunks after the swizzle), computed once and kept in registers.
  uint32_t vlo = (uint32_t)(n * 64 + (((2 * g) ^ v_swz(n)) << 4));
  uint32_t vhi = (uint32_t)(n * 64 + (((2 * g + 1) ^ v_swz(n)) << 4));
  asm volatile("" : "+v"(vlo), "+v"(vhi));
  SoftmaxState st{-INFINITY, kBase0, 0.f};
  v16i biasv;
#pragma unroll
  for (int e = 0; e < 16; ++e) biasv[e] = kBiasBits;
  // Kept resident in 16 registers: without the opaque step the compiler rebuilds the vector
  // with eight 64-bit moves every sub-tile.
  asm volatile("" : "+v"(biasv));
  v16f acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = (v16f){};

  int pending = -1;  // the short sub-tile, done after the loop (it is the last one of the row)
  // Step u: wait for sub-tile u (the older of the two copies in flight), start sub-tile u+2
  // into the buffer sub-tile u-1 used, compute u.
  auto compute = [&](int u, int j, const uint8_t* cur) {
    const int valid = sub_valid(j, u);
    if (valid == 64) {
      if constexpr (F8QK) {
        v16f S[2];
        qk_subtile_f8(cur, qB, n, g, e8m0_code(skh[j]), q_code, S);
        softmax_pv_i8f8<false>(S, cur + kSubBytes, n, g, 64, c_log2, e8m0_code(svh[j]), st, acc, vlo, vhi);
      } else {
        v16i S[2];
        qk_subtile_i8(cur, qB, n, g, S, biasv);
        softmax_pv_i8f8<false>(S, cur + kSubBytes, n, g, 64, (s_q * skh[j]) * c_log2, e8m0_code(svh[j]),
                                st, acc, vlo, vhi);
      }
    } else if (valid > 0) {
      pending = u;
    }
  };
  // Steady state (u + 2 < U): wait for sub-tile u with the copies of u+1 still in flight,
  // start u+2, compute u. No branch guards the waits or the copies, so the compiler's own
  // wait insertion keeps track of which buffer each pending copy targets and adds no wait of
  // its own before the LDS reads.
  auto step = [&](int u, int j, const uint8_t* cur, uint8_t* fill) {
    __builtin_amdgcn_s_waitcnt(0xF70 | kDmaPerTile<NT>);  // u landed, u+1 may fly
    dma_barrier();
    dma(u + 2, fill);
    compute(u, j, cur);
  };
  // The last sub-tiles of the row: the same with the waits and copies the end needs.
  auto last_step = [&](int u, int j, const uint8_t* cur, uint8_t* fill) {
    if (u + 1 < U) __builtin_amdgcn_s_waitcnt(0xF70 | kDmaPerTile<NT>);
    else wait_dma();
    dma_barrier();
    if (u + 2 < U) dma(u + 2, fill);
    compute(u, j, cur);
  };
  dma(0, buf0);
  if (U > 1) dma(1, buf1);
  int u = 0;
  if (u + 4 < U) __builtin_amdgcn_s_waitcnt(0xF70 | kDmaPerTile<NT>);
  for (; u + 4 < U; u += 3) {  // sub-tile u uses buffer u % 3
    const int j0 = blk(u), j1 = blk(u + 1), j2 = blk(u + 2);
    step(u, j0, buf0, buf2);
    step(u + 1, j1, buf1, buf0);
    step(u + 2, j2, buf2, buf1);
    // The next iteration's first wait, done here: on entry to the loop only the copies into
    // buf1 are then in flight, from either edge.
    __builtin_amdgcn_s_waitcnt(0xF70 | kDmaPerTile<NT>);
  }
  // At most four sub-tiles remain (u is a multiple of 3).
  if (u < U) {
    last_step(u, blk(u), buf0, buf2);
    if (u + 1 < U) {
      last_step(u + 1, blk(u + 1), buf1, buf0);
      if (u + 2 < U) {
        last_step(u + 2, blk(u + 2), buf2, buf1);
        if (u + 3 < U) last_step(u + 3, blk(u + 3), buf0, buf2);
      }
    }
  }
  if (pending >= 0) {
    const int jp = blk(pending);
    __syncthreads();
    dma(pending, buf0);
    wait_dma();
    __syncthreads();
    if constexpr (F8QK) {
      v16f S[2];
      qk_subtile_f8(buf0, qB, n, g, e8m0_code(skh[jp]), q_code, S);
      softmax_pv_i8f8<true>(S, buf0 + kSubBytes, n, g, sub_valid(jp, pending), c_log2, e8m0_code(svh[jp]),
                            st, acc, vlo, vhi);
    } else {
      v16i S[2];
      qk_subtile_i8(buf0, qB, n, g, S, biasv);
      softmax_pv_i8f8<true>(S, buf0 + kSubBytes, n, g, sub_valid(jp, pending),
                            (s_q * skh[jp]) * c_log2, e8m0_code(svh[jp]), st, acc, vlo, vhi);
    }
  }
  const float l_tot = st.l;  // row_sum_fp8 covers both key halves of the row
  const float scale = 1.f / l_tot;
  const int64_t row = i * BQ + 32 * wave + n;
  store_out(acc, scale, out + b * ob + h * oh, ol, row, row < L, g);
}

// Debug: the S tile of query block i against key block plan[prow_off] through the attention
// kernel's own MFMA path: exact int32 sums (qk_subtile_i8), or with F8QK the scaled fp32 sums of
// the all-FP8 mode (qk_subtile_f8, both block scales applied by the MFMA). An index outside
// [0, nK) reads block 0.
template <int BQ, bool F8QK>
__global__ __launch_bounds__(BQ * 2) void debug_qk_kernel(const int8_t* __restrict__ Qh,
                                                          const uint8_t* __restrict__ Kh,
                                                          const float* __restrict__ sq,
                                                          const float* __restrict__ sk,
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
    constexpr int kPer = 64 * kD / (16 * NT);
    v4i rk[kPer];
    tile_load<kPer, NT>(rk, Kh + ((bh * nK + j) * nsub + s) * (int64_t)(64 * kD), t);
    __syncthreads();
    tile_store<kPer, NT>(rk, ldsK, t);
    __syncthreads();
    int32_t S[2][16];
    if constexpr (F8QK) {
      v16f F[2];
      qk_subtile_f8(ldsK, qB, n, g, e8m0_code(sk[bh * nK + j]), e8m0_code(sq[bh * nQ + i]), F);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) S[kb][v] = __float_as_int(F[kb][v]);
    } else {
      v16i I[2];
      qk_subtile_i8(ldsK, qB, n, g, I, v16i{});
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) S[kb][v] = I[kb][v];
    }
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
constexpr float kLazyLog2 = 8.f;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
constexpr bf16x2_t kOnesBf16x2 = {(__bf16)1.0f, (__bf16)1.0f};

// S^T and the softmax of one bf16 sub-tile for one wavefront: the weights P (bf16, the B
// operand of the PV product) come back in P; PV follows in pv_bf16 once V^T is in LDS.
template <bool PARTIAL>
__device__ __forceinline__ void qk_softmax_bf16(const uint8_t* ldsK, const v8bf qB[8], int n, int g, int valid,
                                                float c_log2, float& m, float& l, v16f acc[4], v8bf P[4]) {
  v16f S[2];
  {
    // The two key halves' chains interleaved (rows n and n + 32 share the swizzle), with the K
    // fragments of two k steps in flight: each pair is read right after the MFMAs that free
    // its registers (the scheduling barriers keep the compiler from pairing each read with its
    // MFMA; 1 % faster at 480p).
    v16f c0 = {}, c1 = {};
    const uint8_t* base = ldsK + n * (kD * 2);
    const int sw = bk_swz(n);
    auto frag = [&](int kb, int c) { return *(const v8bf*)(base + 32 * kD * 2 * kb + (((2 * c + g) ^ sw) << 4)); };
    v8bf x0 = frag(0, 0), x1 = frag(1, 0), y0 = frag(0, 1), y1 = frag(1, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 8; c += 2) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x0, qB[c], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x1, qB[c], c1, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (c + 2 < 8) {
        x0 = frag(0, c + 2);
        x1 = frag(1, c + 2);
      }
      __builtin_amdgcn_sched_barrier(0);
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(y0, qB[c + 1], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(y1, qB[c + 1], c1, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (c + 3 < 8) {
        y0 = frag(0, c + 3);
        y1 = frag(1, c + 3);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    S[0] = c0;
    S[1] = c1;
  }
  float smax = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      if (PARTIAL && acc_key(kb, v, g) >= valid) S[kb][v] = -INFINITY;
      smax = fmaxf(smax, S[kb][v]);
    }
  smax = xor32_maxf(smax);
  // Lazy rescaling: the reference maximum m only moves when a row's running maximum exceeds it
  // by more than kLazyLog2, so p = 2^(x - m) stays below 2^kLazyLog2 (no fp32/bf16 overflow) and
  // the accumulators are rescaled only on those tiles. The quotient acc / l is unchanged.
  const float m_cand = fmaxf(m, smax * c_log2);
  if (__ballot(m_cand > m + kLazyLog2)) {
    const float alpha = __builtin_amdgcn_exp2f(m - m_cand);  // 0 while m = -inf
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] *= alpha;
    l *= alpha;
    m = m_cand;
  }
  float nm = -m;
  asm("" : "+v"(nm));  // keep the addend a plain VGPR (no negation modifier on every FMA)
  float lsum = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      uint32_t wd[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][8 * hh + e], c_log2, nm));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][8 * hh + e + 1], c_log2, nm));
        wd[e >> 1] = pack_bf16x2(p0, p1);
        // the row sum over the bf16 weights the PV product applies (so they sum to one), two
        // per v_dot2c_f32_bf16 against (1, 1)
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wd[e >> 1]), kOnesBf16x2, lsum, false);
      }
      P[2 * kb + hh] = __builtin_bit_cast(v8bf, make_uint4(wd[0], wd[1], wd[2], wd[3]));
    }
  l += lsum;
}

// O^T += V^T P^T for one bf16 sub-tile (V^T rows of 128 bytes with the bv_swz chunk swizzle).
__device__ __forceinline__ void pv_bf16(const uint8_t* ldsV, const v8bf P[4], int n, int g, v16f acc[4]) {
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int d = 32 * db + n;
    const uint8_t* rowp = ldsV + d * (64 * 2);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int chunk = (2 * kc + g) ^ bv_swz(d);
      const v8bf a = *(const v8bf*)(rowp + chunk * 16);
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, P[kc], acc[db], 0, 0, 0);
    }
  }
}

// bf16 attention: the INT8/FP8 kernel's structure with bf16 operands (16 KB per operand and
// sub-tile). Three workgroups per CU, so three wavefronts per SIMD overlap one another's VALU
// and MFMA work: 168 VGPRs (two values spilled), and 48 KB of LDS with K in two slots and V^T in
// one, refilled after a second barrier in each step.
template <int BQ, int NSUB>
__global__ __launch_bounds__(BQ * 2, 3) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, int64_t qsb, int64_t qsh, int64_t qsl, const int32_t* __restrict__ q_src,
    const uint16_t* __restrict__ qws, const uint8_t* __restrict__ Kt, const uint8_t* __restrict__ Vt,
    const int32_t* __restrict__ plan,
    int64_t H, int L, int64_t nQ, int nK, int n_keep, float c_log2, __bf16* __restrict__ out,
    int64_t ob, int64_t oh, int64_t ol, int64_t total) {
  constexpr int NT = BQ * 2;
  constexpr int kSubBytes = 64 * kD * 2;  // K or V^T bytes of a bf16 sub-tile
  // K double-buffered, V^T single-buffered (48 KB: three workgroups per CU)
  __shared__ __attribute__((aligned(16))) uint8_t bring[3 * kSubBytes];
  uint8_t* const kbuf0 = bring;
  uint8_t* const kbuf1 = bring + kSubBytes;
  uint8_t* const vbuf = bring + 2 * kSubBytes;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63, n = lane & 31, g = lane >> 5;
  const uint32_t wave_lds = __builtin_amdgcn_readfirstlane((uint32_t)wave * 1024u);
  const int64_t w = xcd_remap(blockIdx.x, total);
  const int64_t bh = w / nQ, i = w % nQ;
  const int64_t b = bh / H, h = bh % H;
  const cint32_p prow = (cint32_p)(plan + (bh * nQ + i) * n_keep);
  const uint8_t* Kb = Kt + bh * (int64_t)nK * NSUB * kSubBytes;
  const uint8_t* Vb = Vt + bh * (int64_t)nK * NSUB * kSubBytes;
  const int U = n_keep * NSUB;

  // Q operand: 8 chunks of 8 bf16 (d = 16c + 8g ..) of query row `row`.
  v8bf qB[8];
  const int64_t row = i * BQ + 32 * wave + n;
  {
    // Q from the caller, or (the workspace's Q-source word set by the prologue pass) the
    // normalized, rotated bf16 Q in the workspace, rows [bh][nQ * BQ][128]
    const bool from_ws = *(cint32_p)q_src != 0;
    const uint16_t* qbase = from_ws ? qws + bh * nQ * BQ * kD : q + b * qsb + h * qsh;
    const int64_t ql = from_ws ? (int64_t)kD : qsl;
    const uint16_t* qrow = qbase + (row < L ? row : 0) * ql;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint4 r = make_uint4(0, 0, 0, 0);
      if (row < L) r = *(const uint4*)(qrow + 16 * c + 8 * g);
      qB[c] = __builtin_bit_cast(v8bf, r);
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) settle(qB[c]);
  float cl = c_log2;
  asm("" : "+v"(cl));  // per-lane copy: an SGPR operand would make every exponent FMA a slower VOP3 form

  auto blk = [&](int u) -> int { return prow[(u < U ? u : U - 1) / NSUB]; };
  constexpr int kPer = kSubBytes / (16 * NT);
  static_assert(kPer < 16, "vmcnt immediate 0xF70 | n needs n < 16");
  const uint32_t voff = (uint32_t)t * 16u;
  auto dma_op = [&](const uint8_t* base, int u, uint8_t* dst) {
    int j = blk(u);
    j = (unsigned)j < (unsigned)nK ? j : 0;
    const uint8_t* src = base + ((int64_t)j * NSUB + (u % NSUB)) * kSubBytes;
    const uint32_t lb = lds_addr(dst) + wave_lds;
#pragma unroll
    for (int k = 0; k < kPer; ++k) lds_dma16(src + k * NT * 16, voff, lb + k * NT * 16);
  };
  auto sub_valid = [&](int j, int u) -> int {
    return (unsigned)j < (unsigned)nK ? min(64, L - (j * (64 * NSUB) + 64 * (u % NSUB))) : 0;
  };
  float m = -INFINITY, l = 0.f;
  v16f acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = (v16f){};

  // Step u: wait for K(u), barrier (every wavefront is done with step u-1, so the V^T buffer and
  // the other K buffer are free), copy V^T(u) and then K(u+1), QK^T and softmax of u, wait for
  // V^T(u) (K(u+1) may stay in flight), barrier, PV of u.
  int pending = -1;
  auto step = [&](int u, int j, const uint8_t* kcur, uint8_t* knext) {
    wait_dma();
    dma_barrier();
    dma_op(Vb, u, vbuf);
    if (u + 1 < U) dma_op(Kb, u + 1, knext);
    const int valid = sub_valid(j, u);
    v8bf P[4];
    if (valid == 64) qk_softmax_bf16<false>(kcur, qB, n, g, 64, cl, m, l, acc, P);
    if (u + 1 < U) __builtin_amdgcn_s_waitcnt(0xF70 | kPer);
    else wait_dma();
    dma_barrier();
    if (valid == 64) pv_bf16(vbuf, P, n, g, acc);
    else if (valid > 0) pending = u;
  };
  dma_op(Kb, 0, kbuf0);
  for (int u = 0; u < U; u += 2) {
    const int j0 = blk(u), j1 = blk(u + 1);
    step(u, j0, kbuf0, kbuf1);
    if (u + 1 < U) step(u + 1, j1, kbuf1, kbuf0);
  }
  if (pending >= 0) {
    const int jp = blk(pending);
    __syncthreads();
    dma_op(Kb, pending, kbuf0);
    dma_op(Vb, pending, vbuf);
    wait_dma();
    __syncthreads();
    v8bf P[4];
    qk_softmax_bf16<true>(kbuf0, qB, n, g, sub_valid(jp, pending), cl, m, l, acc, P);
    pv_bf16(vbuf, P, n, g, acc);
  }
  const float l_tot = xor32_sum(l);
  store_out(acc, 1.f / l_tot, out + b * ob + h * oh, ol, row, row < L, g);
}

// ---------------------------------------------------------------------------------------
void launch_attend_i8f8(const sa_forward_layout& lay, const char* ws, const int32_t* plan,
                        int64_t B, int64_t H, int64_t L, int bq, int bk, int64_t n_keep,
                        float c_log2, bool qk_fp8, const TensorView& out, hipStream_t s) {
  const int64_t total = B * H * lay.nQ;
  const int8_t* Qh = (const int8_t*)(ws + lay.q_off);
  const uint8_t* Kh = (const uint8_t*)(ws + lay.k_off);
  const uint8_t* Vt = (const uint8_t*)(ws + lay.v_off);
  const float* sq = (const float*)(ws + lay.sq_off);
  const float* sk = (const float*)(ws + lay.sk_off);
  const float* sv = (const float*)(ws + lay.sv_off);
  __bf16* o = (__bf16*)out.data;
  const unsigned grid = (unsigned)total;
#define SA_LAUNCH_I8(BQ, NSUB, F8)                                                                 \
  attn_i8f8_kernel<BQ, NSUB, F8><<<grid, BQ * 2, 0, s>>>(Qh, Kh, Vt, sq, sk, sv, plan, H, (int)L,      \
                                                         lay.nQ, (int)lay.nK, (int)n_keep, c_log2, o, \
                                                         out.sb, out.sh, out.sl, total)
  if (qk_fp8) {
    if (bq == 128 && bk == 64) SA_LAUNCH_I8(128, 1, true);
    else if (bq == 128) SA_LAUNCH_I8(128, 2, true);
    else if (bk == 64) SA_LAUNCH_I8(64, 1, true);
    else SA_LAUNCH_I8(64, 2, true);
  } else {
    if (bq == 128 && bk == 64) SA_LAUNCH_I8(128, 1, false);
    else if (bq == 128) SA_LAUNCH_I8(128, 2, false);
    else if (bk == 64) SA_LAUNCH_I8(64, 1, false);
    else SA_LAUNCH_I8(64, 2, false);
  }
#undef SA_LAUNCH_I8
}

void launch_attend_bf16(const TensorView& q, const sa_forward_layout& lay, const char* ws,
                        const int32_t* plan, int64_t B, int64_t H, int64_t L, int bq, int bk,
                        int64_t n_keep, float c_log2, const TensorView& out, hipStream_t s) {
  const int64_t total = B * H * lay.nQ;
  const uint8_t* Kt = (const uint8_t*)(ws + lay.k_off);
  const uint8_t* Vt = (const uint8_t*)(ws + lay.v_off);
  __bf16* o = (__bf16*)out.data;
  const uint16_t* qd = (const uint16_t*)q.data;
  const int32_t* qsrc = (const int32_t*)(ws + lay.sq_off);
  const uint16_t* qws = (const uint16_t*)(ws + lay.q_off);
  const unsigned grid = (unsigned)total;
#define SA_LAUNCH_BF(BQ, NSUB)                                                                    \
  attn_bf16_kernel<BQ, NSUB><<<grid, BQ * 2, 0, s>>>(qd, q.sb, q.sh, q.sl, qsrc, qws, Kt, Vt, plan, H, (int)L, \
                                                     lay.nQ, (int)lay.nK, (int)n_keep, c_log2, o,    \
                                                     out.sb, out.sh, out.sl, total)
  if (bq == 128 && bk == 64) SA_LAUNCH_BF(128, 1);
  else if (bq == 128) SA_LAUNCH_BF(128, 2);
  else if (bk == 64) SA_LAUNCH_BF(64, 1);
  else SA_LAUNCH_BF(64, 2);
#undef SA_LAUNCH_BF
}

void launch_debug_qk(const sa_forward_layout& lay, const char* ws, const int32_t* plan, int64_t B,
                     int64_t H, int64_t L, int bq, int bk, int64_t n_keep, int64_t b, int64_t h,
                     int64_t i, int64_t t, bool qk_fp8, void* out, hipStream_t s) {
  (void)B; (void)L;
  const int nsub = bk / 64;
  const int64_t prow_off = ((b * H + h) * lay.nQ + i) * n_keep + t;
  const int8_t* Qh = (const int8_t*)(ws + lay.q_off);
  const uint8_t* Kh = (const uint8_t*)(ws + lay.k_off);
  const float* sq = (const float*)(ws + lay.sq_off);
  const float* sk = (const float*)(ws + lay.sk_off);
  int32_t* o = (int32_t*)out;
#define SA_LAUNCH_DBG(BQ, F8) \
  debug_qk_kernel<BQ, F8><<<1, BQ * 2, 0, s>>>(Qh, Kh, sq, sk, plan, prow_off, lay.nQ, lay.nK, nsub, b * H + h, i, o)
  if (bq == 128) {
    if (qk_fp8) SA_LAUNCH_DBG(128, true);
    else SA_LAUNCH_DBG(128, false);
  } else {
    if (qk_fp8) SA_LAUNCH_DBG(64, true);
    else SA_LAUNCH_DBG(64, false);
  }
#undef SA_LAUNCH_DBG
}

}  // namespace sa
