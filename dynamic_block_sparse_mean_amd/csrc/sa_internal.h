// Internal declarations shared by the library's translation units (host and device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparse_attn.h"

namespace sa {

// ---- vector types for MFMA operands ----------------------------------------
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kD = 128;          // head dimension supported
constexpr int kSub = 64;         // keys per attention sub-tile
constexpr int kMaxKeyBlocks = 4096;

// 16-byte chunk swizzles of the attention tiles, chosen so that a 16-lane group of a
// ds_read_b128 (256 bytes, all 64 LDS banks) reads 16 distinct bank groups: chunk c of row r
// is stored at c ^ swz(r). INT8/FP8: K^ rows of 128 bytes (8 chunks; rows r and r + 1 share
// a 256-byte bank line), V^T rows of 64 bytes (4 chunks, four rows per bank line).
__host__ __device__ constexpr int k_swz(int r) { return (r >> 1) & 7; }
__host__ __device__ constexpr int v_swz(int d) { return (d >> 2) & 3; }
// bf16 tiles: K rows of 256 bytes (16 chunks), V^T rows of 128 bytes (8 chunks).
__host__ __device__ constexpr int bk_swz(int r) { return r & 15; }
__host__ __device__ constexpr int bv_swz(int d) { return (d >> 1) & 7; }

// ---- error reporting (host) -------------------------------------------------
int set_error(int status, const char* fmt, ...);
int check_launch(const char* what);

// ---- device tensor view -----------------------------------------------------
struct TensorView {
  const void* data;
  int dtype;
  int64_t sb, sh, sl;
};

// ---- division by a launch constant --------------------------------------------
// n / d for 0 <= n < 2^31 and 1 <= d < 2^31 by multiply and shift: (n * m) >> k with
// k = 31 + ceil(log2 d) and m = floor(2^k / d) + 1 (m < 2^32). Exact: with m = 2^k/d + e,
// 0 < e <= 1, the quotient is n/d + n e / 2^k and n e / 2^k < 2^-ceil(log2 d) <= 1/d, too
// little to reach the next multiple of d. Workgroup ids stay below 2^24 on this path, so the
// kernels split their id into (batch, head, block) this way instead of with 64-bit divisions
// (hundreds of scalar instructions ahead of the first load of a short-lived workgroup).
struct DivMagic {
  uint32_t d, m, k;
};
inline DivMagic div_magic_for(uint32_t d) {
  uint32_t lg = 0;
  while (((uint64_t)1 << lg) < d) ++lg;
  const uint32_t k = 31 + lg;
  return DivMagic{d, (uint32_t)(((uint64_t)1 << k) / d + 1), k};
}
__device__ __forceinline__ uint32_t div_magic(uint32_t n, uint32_t m, uint32_t k) {
  return (uint32_t)(((uint64_t)n * m) >> k);
}
__device__ __forceinline__ uint32_t div_magic(uint32_t n, const DivMagic& dm) { return div_magic(n, dm.m, dm.k); }

// ---- streaming loads -------------------------------------------------------------
// 16 bytes of an input read once (nontemporal hint: the line is not kept for reuse in the
// caches). The pooling pass runs 8-10 % faster with it; the quantization pass about 0.7 %.
__device__ __forceinline__ uint4 load_stream(const void* p) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const u4 x = __builtin_nontemporal_load((const u4*)p);
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// ---- XCD-aware work mapping --------------------------------------------------
// Workgroups are handed to the 8 XCDs round-robin by workgroup id. Remap so that each
// XCD works on a contiguous range of logical work items: neighbouring query blocks of
// one head (which keep overlapping key blocks) then share that XCD's L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t w, int64_t total) {
  const int64_t q = total >> 3, r = total & 7;
  const int64_t x = w & 7, s = w >> 3;
  return x * q + (x < r ? x : r) + s;
}

// ---- wave-level helpers -------------------------------------------------------
__device__ __forceinline__ double wave_max_f64(double v) {
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ double wave_min_f64(double v) {
  for (int o = 32; o > 0; o >>= 1) v = fmin(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_sum_i32(int v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max_f32(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// exclusive prefix sum over the 64 lanes
__device__ __forceinline__ int wave_excl_scan_i32(int v, int lane) {
  int x = v;
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x - v;
}

// ---- launchers (one per translation unit) -------------------------------------
void launch_pool(const TensorView& x, int64_t B, int64_t H, int64_t L, int block,
                 double* means, hipStream_t s);
void launch_scores(const double* qm, const double* km, int64_t BH, int64_t nQ, int64_t nK,
                   double* scores, hipStream_t s);
void launch_topk(const double* scores, int64_t rows, int64_t nK, int64_t n_keep,
                 int32_t* plan, hipStream_t s);
// RMSNorm + 3-D RoPE of Q and K ahead of the block means and the quantization.
struct QkPrologue {
  const float* q_gain;  // fp32 [H][128]
  const float* k_gain;  // fp32 [H][128]
  float eps;            // > 0 (the caller's eps rounded to fp32)
  int64_t grid_t, grid_h, grid_w;
  double theta;
  float2* table;        // rope_table_bytes(...) of device memory (written by launch_quant)
  // set by launch_quant: division by grid_h * grid_w and by grid_w
  DivMagic hw, w;
};
size_t rope_table_bytes(int64_t T, int64_t Hg, int64_t Wg);

// qmeans/kmeans: when not null, also write the fp64 block means of Q and K (the pooling
// step of the plan) from the same pass over the inputs. pro: when not null, Q and K pass
// through the prologue first (its rotary table is computed into pro->table on the stream).
void launch_quant(const TensorView& q, const TensorView& k, const TensorView& v,
                  int64_t B, int64_t H, int64_t L, int bq, int bk, const sa_forward_layout& lay,
                  char* ws, double* qmeans, double* kmeans, bool qk_fp8, const QkPrologue* pro,
                  hipStream_t s);
void launch_layout_bf16(const TensorView& k, const TensorView& v, int64_t B, int64_t H,
                        int64_t L, int bk, const sa_forward_layout& lay, char* ws, hipStream_t s);
// bf16 mode with the prologue: normalized, rotated Q (bf16) into the workspace's Q region and K
// into the K tiles, their fp64 block means into qmeans/kmeans, V laid out as without it; the
// workspace's Q-source word is set so that the bf16 attention reads that Q.
void launch_prologue_bf16(const TensorView& q, const TensorView& k, const TensorView& v, int64_t B,
                          int64_t H, int64_t L, int bq, int bk, const sa_forward_layout& lay, char* ws,
                          double* qmeans, double* kmeans, const QkPrologue& pro, hipStream_t s);
// qk_fp8: Q^ and K^ hold E4M3 codes with power-of-two scales (all-FP8 mode) instead of INT8.
void launch_attend_i8f8(const sa_forward_layout& lay, const char* ws, const int32_t* plan,
                        int64_t B, int64_t H, int64_t L, int bq, int bk, int64_t n_keep,
                        float c_log2, bool qk_fp8, const TensorView& out, hipStream_t s);
void launch_attend_bf16(const TensorView& q, const sa_forward_layout& lay, const char* ws,
                        const int32_t* plan, int64_t B, int64_t H, int64_t L, int bq, int bk,
                        int64_t n_keep, float c_log2, const TensorView& out, hipStream_t s);
// Light-Ulysses FP8 payload: pack (tensors -> payload) or unpack (payload -> tensors) of t[0..T).
//   head_side: the tensors hold the hc heads of a head chunk over the whole sequence (limit = L);
//   otherwise they hold one token shard of all heads (limit = the shard's length), and the chunk is
//   heads [h0, h0 + hc) of each group of `group` heads.
void launch_ulysses(bool pack, const TensorView* t, int T, bool head_side, int64_t B, int64_t lmax, int64_t hc,
                    int64_t group, int64_t h0, int64_t limit, int peers, int64_t chunk_bytes, uint8_t* payload,
                    hipStream_t s);
// NVFP4: quantize a bf16 [R][K] matrix (row stride ld) into codes [R][K/2], E4M3 block scales
// [R][K/16] and the fp32 tensor scale S (partial: nparts floats of scratch); GEMM of two NVFP4
// matrices, Y[m][n] = S_A S_W sum_k (q_A s_A)(q_W s_W) + bias[n] in bf16 (row stride ldy).
constexpr int kNvfp4Parts = 1024;
void launch_nvfp4_quantize(const uint16_t* x, int64_t R, int64_t K, int64_t ld, uint8_t* codes, uint8_t* scales,
                           float* S, float* partial, int nparts, hipStream_t s);
void launch_nvfp4_gemm(const uint8_t* A, const uint8_t* As, const float* SA, const uint8_t* W, const uint8_t* Ws,
                       const float* SW, const uint16_t* bias, uint16_t* Y, int M, int N, int K, int64_t ldy,
                       hipStream_t s);
// out: int32 [bq][bk] (INT8 tiles) or fp32 [bq][bk] (qk_fp8: scaled FP8 scores)
void launch_debug_qk(const sa_forward_layout& lay, const char* ws, const int32_t* plan,
                     int64_t B, int64_t H, int64_t L, int bq, int bk, int64_t n_keep,
                     int64_t b, int64_t h, int64_t i, int64_t t, bool qk_fp8, void* out, hipStream_t s);

}  // namespace sa
