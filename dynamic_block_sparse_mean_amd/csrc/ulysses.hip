// Light-Ulysses FP8 packing: the single-GPU part of the sequence-parallel path.
//
// Page "600倍加速，720p视频实时生成！单卡也能带的动14B模型", multi-card path, Light-Ulysses
// paragraph; page "600 倍加速 720p 视频实时生成 — 单卡 14B 模型推理优化", the memory and
// communication item of its summary; page "Run Wan2.2-A14B on One RTX 5090: 720p Video in 3.8s",
// section 4: the token sequence is split over the GPUs and an all-to-all moves Q, K, V from the
// sequence split to a head split before attention, and the output back after it; the data
// travels in FP8 both ways, Q, K and V travel as one payload prepared by fused pre- and
// post-processing kernels, and the exchange is pipelined by groups of heads (the next heads move
// while the current ones compute). These are those kernels; the all-to-all itself is the
// caller's collective.
//
// Readings (the pages give no format): P peers; tokens in P contiguous shards of Lmax = ceil(L/P)
// (the last one shorter), heads in P contiguous groups of H/P. Every row of 128 values (one token,
// one head, one tensor) goes as E4M3 codes with one power-of-two scale 2^e (e the smallest integer
// with max|row| <= 448 * 2^e, clamped to [-127, 127], 0 for a zero row), sent as the byte 127 + e.
// A head chunk [h0, h0 + hc) of every group travels as a payload of its own (hc = H/P: all heads).
// The payload is P equal chunks, one per destination (sender side) or per source (receiver
// side); chunk c = codes [B][Lmax][hc][T][128], then one scale byte per row, [B][Lmax][hc][T],
// then padding up to a multiple of 256 bytes. Rows past the end of a short shard: code 0, e = 0.
//
// HBM-bound: 8 lanes per row, 16-byte loads and stores on both sides.
#include "sa_internal.h"

namespace sa {

// Payload row (c, b, t, hl, ti) -> (head, token) of a tensor on one side of the exchange.
//   head side (the peer that holds whole sequences of its head chunk): the tensor has the
//       chunk's hc heads; head hl, token c * lmax + t, present while < limit (= L);
//   sequence side (the peer that holds one token shard of all H heads): head c * group + h0 + hl,
//       token t, present while < limit (= the shard's length).
struct UlyssesMap {
  int64_t lmax, hc, group, h0, limit;
  bool head_side;
  __device__ __forceinline__ bool row(int64_t c, int64_t t, int64_t hl, int64_t* h, int64_t* n) const {
    *h = head_side ? hl : c * group + h0 + hl;
    *n = head_side ? c * lmax + t : t;
    return *n < limit;
  }
};

struct UlyssesTensors {
  void* data[3];
  int64_t sb[3], sh[3], sl[3];
};

struct UlyssesPayload {
  uint8_t* base;
  int64_t rows;   // rows per chunk: B * lmax * hc * T
  int64_t chunk;  // bytes per chunk
  __device__ __forceinline__ uint8_t* codes(int64_t c, int64_t i) const { return base + c * chunk + i * kD; }
  __device__ __forceinline__ uint8_t* scale(int64_t c, int64_t i) const { return base + c * chunk + rows * kD + i; }
};

// Work split: 8 lanes per row (16 values each), 32 rows per pass of a 256-thread workgroup and
// kRows passes per workgroup, every load of a thread issued before any of its arithmetic. The
// grid's y index is the slab (c, b) (uniform per workgroup); x covers the slab's Lmax * hc * T
// rows with 32-bit index arithmetic. Rows are handed out token-fastest, so one pass touches 32
// consecutive tokens of one head and tensor (8 KB of contiguous bf16) and 128-byte payload rows
// at a fixed stride. The token-fastest order measured faster than the payload-order walk in both
// directions; pack's payload stores are streaming (nontemporal: plain stores made it 19 % slower),
// unpack's tensor stores plain (nontemporal ones made it 2-16 % slower).
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
constexpr int kLanes = 8, kRowsPerPass = 256 / kLanes, kRows = 2;

struct RowIndex {
  int64_t c, i, b;
  uint32_t t, hl;
  int ti;
  bool live;
};
template <int T>
__device__ __forceinline__ RowIndex row_index(const UlyssesMap& m, int64_t B, int u) {
  RowIndex r;
  const uint32_t hc = (uint32_t)m.hc, lmax = (uint32_t)m.lmax, slab = lmax * hc * T;
  const uint32_t k = (blockIdx.x * kRows + u) * kRowsPerPass + threadIdx.x / kLanes;
  r.live = k < slab;
  const uint32_t c = blockIdx.y / (uint32_t)B;
  r.c = c;
  r.b = blockIdx.y - c * (uint32_t)B;
  const uint32_t th = k / lmax;  // (ti, hl) group of the row
  r.t = k - th * lmax;
  r.ti = (int)(th / hc);
  r.hl = th - (uint32_t)r.ti * hc;
  r.i = r.b * slab + ((int64_t)r.t * hc + r.hl) * T + r.ti;
  return r;
}

__device__ __forceinline__ float max8(float m) {
  // max over the 8 lanes that share a row (lanes 8k .. 8k + 7)
#pragma unroll
  for (int o = 4; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  return m;
}

// E4M3 codes of 16 bf16 values (two uint4 words) under the row's shared scale; returns the scale byte.
__device__ __forceinline__ uint32_t quantize16(const uint4 (&raw)[2], uint4* codes) {
  float f[16];
  float amax = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t w[4] = {raw[h].x, raw[h].y, raw[h].z, raw[h].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[8 * h + 2 * e] = __uint_as_float(w[e] << 16);
      f[8 * h + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(f[e]));
  amax = max8(amax);
  // amax = fr * 2^k2 with fr in [0.5, 1): amax <= 448 * 2^e  <=>  e >= k2 - 9 + (fr > 0.875)
  int k2;
  const float fr = frexpf(amax, &k2);
  int ex = fr <= 0.875f ? k2 - 9 : k2 - 8;
  ex = amax > 0.f ? min(max(ex, -127), 127) : 0;
  const float inv = ldexpf(1.f, -ex);
  uint32_t packed[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = fminf(fmaxf(f[4 * q + e] * inv, -448.f), 448.f);
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    packed[q] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
  }
  *codes = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  return (uint32_t)(127 + ex);
}

template <int T>
__global__ __launch_bounds__(256) void ulysses_pack_kernel(UlyssesTensors x, UlyssesMap map, int64_t B,
                                                           UlyssesPayload pay) {
  const int j = threadIdx.x % kLanes;  // values 16j .. 16j+15 of the row
  RowIndex r[kRows];
  uint4 raw[kRows][2];
#pragma unroll
  for (int u = 0; u < kRows; ++u) {
    r[u] = row_index<T>(map, B, u);
    raw[u][0] = raw[u][1] = make_uint4(0, 0, 0, 0);
    int64_t h, n;
    if (r[u].live && map.row(r[u].c, r[u].t, r[u].hl, &h, &n)) {
      const int ti = r[u].ti;
      const uint4* src =
          (const uint4*)((const uint16_t*)x.data[ti] + r[u].b * x.sb[ti] + h * x.sh[ti] + n * x.sl[ti] + 16 * j);
      raw[u][0] = src[0];
      raw[u][1] = src[1];
    }
  }
#pragma unroll
  for (int u = 0; u < kRows; ++u) {
    if (!r[u].live) break;  // rows past the slab come last; the 8 lanes of a row agree
    uint4 codes;
    const uint32_t sbyte = quantize16(raw[u], &codes);
    const v4u cv = {codes.x, codes.y, codes.z, codes.w};
    __builtin_nontemporal_store(cv, (v4u*)(pay.codes(r[u].c, r[u].i) + 16 * j));
    if (j == 0) *pay.scale(r[u].c, r[u].i) = (uint8_t)sbyte;
  }
}

__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const f2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2));
}

template <int T>
__global__ __launch_bounds__(256) void ulysses_unpack_kernel(UlyssesPayload pay, UlyssesMap map, int64_t B,
                                                             UlyssesTensors y) {
  const int j = threadIdx.x % kLanes;
  RowIndex r[kRows];
  uint4 cw[kRows];
  int ex[kRows];
  bool store[kRows];
  int64_t h[kRows], n[kRows];
#pragma unroll
  for (int u = 0; u < kRows; ++u) {
    r[u] = row_index<T>(map, B, u);
    // a padding row of a short shard is not written
    store[u] = r[u].live && map.row(r[u].c, r[u].t, r[u].hl, &h[u], &n[u]);
    if (store[u]) {
      cw[u] = *(const uint4*)(pay.codes(r[u].c, r[u].i) + 16 * j);
      ex[u] = (int)*pay.scale(r[u].c, r[u].i) - 127;
    }
  }
#pragma unroll
  for (int u = 0; u < kRows; ++u) {
    if (!store[u]) continue;
    const uint32_t w[4] = {cw[u].x, cw[u].y, cw[u].z, cw[u].w};
    uint32_t out[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // E4M3 -> fp32 and the scale 2^e are exact; the bf16 rounding is exact too unless the value
      // falls below bf16's smallest subnormal.
      typedef float f2 __attribute__((ext_vector_type(2)));
      const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w[q], false);
      const f2 c = __builtin_amdgcn_cvt_pk_f32_fp8(w[q], true);
      out[2 * q] = bf16x2_rne(ldexpf(a[0], ex[u]), ldexpf(a[1], ex[u]));
      out[2 * q + 1] = bf16x2_rne(ldexpf(c[0], ex[u]), ldexpf(c[1], ex[u]));
    }
    const int ti = r[u].ti;
    uint4* dst = (uint4*)((uint16_t*)y.data[ti] + r[u].b * y.sb[ti] + h[u] * y.sh[ti] + n[u] * y.sl[ti] + 16 * j);
    const v4u o0 = {out[0], out[1], out[2], out[3]}, o1 = {out[4], out[5], out[6], out[7]};
    *(v4u*)dst = o0;
    *((v4u*)dst + 1) = o1;
  }
}

void launch_ulysses(bool pack, const TensorView* t, int T, bool head_side, int64_t B, int64_t lmax, int64_t hc,
                    int64_t group, int64_t h0, int64_t limit, int peers, int64_t chunk_bytes, uint8_t* payload,
                    hipStream_t s) {
  UlyssesTensors x{};
  for (int i = 0; i < T; ++i) {
    x.data[i] = const_cast<void*>(t[i].data);
    x.sb[i] = t[i].sb;
    x.sh[i] = t[i].sh;
    x.sl[i] = t[i].sl;
  }
  const UlyssesMap map{lmax, hc, group, h0, limit, head_side};
  const UlyssesPayload pay{payload, B * lmax * hc * T, chunk_bytes};
  const int64_t per_wg = (int64_t)kRowsPerPass * kRows;
  const dim3 grid((unsigned)((lmax * hc * T + per_wg - 1) / per_wg), (unsigned)(peers * B));
#define SA_ULYSSES(TT)                                                          \
  if (pack) ulysses_pack_kernel<TT><<<grid, 256, 0, s>>>(x, map, B, pay);      \
  else ulysses_unpack_kernel<TT><<<grid, 256, 0, s>>>(pay, map, B, x);
  switch (T) {
    case 1: SA_ULYSSES(1) break;
    case 2: SA_ULYSSES(2) break;
    default: SA_ULYSSES(3) break;
  }
#undef SA_ULYSSES
}

}  // namespace sa
