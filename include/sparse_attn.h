/*
 * sparse_attn.h - C ABI of the block-sparse attention library for AMD MI355X (gfx950).
 *
 * What it computes. Self-attention over a long token sequence where each block of
 * block_q consecutive query tokens attends only to a few key blocks of block_k
 * tokens, chosen at run time from block means of Q and K:
 *   1. pool   - mean of Q over each query block and of K over each key block;
 *   2. score  - dot product of every query-block mean with every key-block mean;
 *   3. select - per query block, the n_keep highest-scoring key blocks;
 *   4. quantize (quantized modes) - Q and K to INT8 (or FP8 E4M3 in the all-FP8 mode),
 *                 V to FP8 E4M3, one scale per (batch, head, block);
 *   5. attend - softmax attention of each query over the keys of its kept blocks,
 *                 dense inside every kept tile, online softmax in fp32.
 * Sources: page "600倍加速，720p视频实时生成！单卡也能带的动14B模型" (66bd.net), single-card
 * path, paragraphs on dynamic sparse quantized attention (block means of Q/K, run-time
 * choice of key blocks, only activated tiles computed, dense inside them, 10-20 % of
 * blocks kept) and on efficient inference operators (about 10 % kept, Q/K in INT8 and
 * V in FP8); page "Run Wan2.2-A14B on One RTX 5090: 720p Video in 3.8s", section
 * "3. Dynamic sparse attention". The pages give no formula; the readings taken where
 * they are silent are stated at each call below.
 *
 * Conventions for every call:
 *   - Return SA_OK (0) or a negative status. On error nothing is enqueued and
 *     sa_last_error() (thread-local) says why. No exception crosses the ABI.
 *   - Every pointer to tensor data is a device pointer owned by the caller. The
 *     library allocates, frees and synchronises nothing; work is enqueued on the
 *     caller's stream (0 = the null stream) and faults surface at the caller's
 *     next synchronisation.
 *   - Reentrant; no global state beyond the loaded code object.
 *   - Supported: D = 128, block_q in {64, 128}, block_k in {64, 128},
 *     ceil(L/block_k) <= 4096, inputs bf16 (fp32 accepted by pool/plan); one launch
 *     holds B*H <= 65535 and B*H*(nQ + 2 nK) <= 16777215 (nQ, nK the query and key
 *     block counts). Outside these, SA_ERR_UNSUPPORTED before anything is enqueued.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
enum {
  SA_OK = 0,
  SA_ERR_INVALID_ARG = -1,   /* null pointer, non-positive size, keep not in (0,1] */
  SA_ERR_UNSUPPORTED = -2,   /* D != 128, block size, dtype, stride of d != 1, too large */
  SA_ERR_WORKSPACE = -3,     /* workspace null or smaller than the sizing call says */
  SA_ERR_SHAPE_MISMATCH = -4,/* q/k/v/out/plan shapes disagree */
  SA_ERR_HIP = -5            /* a HIP launch failed; sa_last_error() has the message */
};

enum { SA_DTYPE_FP32 = 0, SA_DTYPE_BF16 = 1 };

/* Attention arithmetic: bf16 MFMA with P in bf16; INT8 QK^T + FP8 PV; or all-FP8 (Q and K
 * also in E4M3, with power-of-two block scales like V: the FP8 sparse attention path the
 * pages name, read with Q/K in FP8 too). The two quantized modes share the workspace layout. */
enum { SA_MODE_BF16 = 0, SA_MODE_INT8_FP8 = 1, SA_MODE_FP8 = 2 };

/* A strided view of a logical [B, H, L, D] tensor in device memory (caller-owned).
 * Strides are in elements; the stride of D must be 1, so both [B,H,L,D] and
 * [B,L,H,D] storage work. */
typedef struct sa_tensor {
  void* data;
  int32_t dtype;     /* SA_DTYPE_* */
  int32_t reserved;  /* must be 0 */
  int64_t B, H, L, D;
  int64_t stride_b, stride_h, stride_l;
} sa_tensor;

/* Byte offsets of the pieces of the forward workspace (see sa_forward_workspace_layout). */
typedef struct sa_forward_layout {
  int64_t nQ, nK;       /* ceil(L/block_q), ceil(L/block_k) */
  size_t q_off;         /* quantized modes: Q^ int8 or E4M3 [B*H][nQ][block_q][D], row-major, pad rows 0;
                           bf16 mode: the prologue's normalized, rotated Q in bf16, same shape (written
                           only by sparse_attn_plan_prepare_prologue) */
  size_t k_off;         /* K^ int8 or E4M3 / K bf16 [B*H][nK][block_k/64][64][D], 16-byte chunk c of
                           row r stored at chunk position c ^ ((r >> 1) & 7) (int8, E4M3) or
                           c ^ (r & 15) (bf16), pad rows 0 */
  size_t v_off;         /* V^T fp8 / V^T bf16 [B*H][nK][block_k/64][D][64]: row d holds the
                           64 keys of a sub-tile in MFMA operand order, 16-byte chunks
                           swizzled (fp8: c ^ ((d >> 2) & 3); bf16: c ^ ((d >> 1) & 7)), pad 0 */
  size_t sq_off;        /* fp32 [B*H][nQ]  Q block scales (quantized modes; powers of two in FP8 mode);
                           bf16 mode: one int32, 1 when q_off holds the prologue's Q (the bf16 attention
                           then reads Q there), 0 after sparse_attn_prepare (it reads q) */
  size_t sk_off;        /* fp32 [B*H][nK]  K block scales (quantized modes; powers of two in FP8 mode) */
  size_t sv_off;        /* fp32 [B*H][nK]  V block scales (quantized modes; always powers of two) */
  size_t total;         /* bytes the caller must provide */
} sa_forward_layout;

/* ---- errors and sizes (host only, no GPU work) -------------------------- */
const char* sa_status_string(int status);
/* Message of the last failing call on this thread ("" if none). */
const char* sa_last_error(void);

/* ceil(L / block); -1 if an argument is not positive. */
int64_t sa_num_blocks(int64_t L, int64_t block);

/* Key blocks kept per query block: min(nK, max(1, ceil(keep_ratio*nK - 1e-6))).
 * Reading of the pages' "keep 10-20 % of the blocks": every query-block row keeps the
 * same count, computed in double precision (a float32 0.1 would give 193 of 1920).
 * Returns -1 if nK < 1 or keep_ratio is not in (0, 1]. */
int64_t sa_plan_n_keep(int64_t nK, double keep_ratio);

/* Workspace of sparse_attn_plan: block means (fp64) and the pooled score matrix
 * (fp64 [B*H][nQ][nK]). */
int sa_plan_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t D,
                            int block_q, int block_k, size_t* bytes);

/* Workspace of sparse_attn_forward / prepare / attend for a mode, and its layout. */
int sa_forward_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t D,
                               int block_q, int block_k, int mode, size_t* bytes);
int sa_forward_workspace_layout(int64_t B, int64_t H, int64_t L, int64_t D,
                                int block_q, int block_k, int mode, sa_forward_layout* layout);

/* Scratch limit of sparse_attn_plan_noalloc, in bytes (64 MiB): shapes whose
 * sa_plan_workspace_bytes exceeds it are rejected by that call. */
#define SA_PLAN_NOALLOC_MAX_BYTES ((size_t)64 << 20)

/* ---- the two calls of the method ------------------------------------------ */

/* Block plan: pool (block means of Q over block_q tokens and of K over block_k tokens,
 * per (batch, head), fp64 sums; a short last block is averaged over its own tokens),
 * score (Qbar . Kbar in fp64, unscaled), select (per query block the n_keep largest
 * scores, equal scores to the lower block index) - the estimate-then-select step of
 * the pages' method.
 *   q, k      : bf16 or fp32, same B, H, L, D.
 *   plan_idx  : device int32 [B][H][nQ][plan_n_keep], written with each row ascending.
 *   plan_n_keep must equal sa_plan_n_keep(nK, keep_ratio) (guards the allocation).
 *   workspace : >= sa_plan_workspace_bytes(...) bytes of device memory. */
int sparse_attn_plan(const sa_tensor* q, const sa_tensor* k, int block_q, int block_k,
                     double keep_ratio, int32_t* plan_idx, int64_t plan_n_keep,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Block-sparse attention over a plan: prepare (INT8/FP8 mode: per-block symmetric INT8
 * of Q and K with s = amax/127 (fp32), FP8 E4M3 of V with the power-of-two scale 2^e,
 * e the smallest integer with amax <= 448 * 2^e, RNE; FP8 mode: Q and K like V; BF16 mode:
 * tile layout of K and V)
 * then attend: for every query block, for each kept key block in ascending order, taken
 * as tiles of 64 keys, S = Q K^T (exact int32 in INT8 mode), online softmax in fp32
 * (log2 domain), P in FP8 (x 2^8) or bf16, O += P V; finally O = acc / rowsum, written
 * as bf16. No causal mask; keys outside the kept blocks get weight 0.
 *   q, k, v   : bf16, same shape; out: bf16, same shape as q (may not alias inputs).
 *   plan_idx  : device int32 [B][H][nQ][n_keep], rows ascending; an entry outside
 *               [0, nK) is skipped (its tile contributes no keys).
 *   sm_scale  : softmax scale; <= 0 selects 1/sqrt(D).
 *   workspace : >= sa_forward_workspace_bytes(..., mode) bytes. */
int sparse_attn_forward(const sa_tensor* q, const sa_tensor* k, const sa_tensor* v,
                        const int32_t* plan_idx, int block_q, int block_k, int64_t n_keep,
                        int mode, float sm_scale, const sa_tensor* out,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* sparse_attn_plan followed by sparse_attn_prepare, with one pass over the inputs: in
 * the quantized modes the quantization pass also takes the block means of Q and K, so Q and K
 * are read once instead of twice (the plan and the workspace are bit-identical to those
 * of the two separate calls). In BF16 mode the two calls are made as they are.
 *   q, k, v       : bf16, same shape.
 *   plan_idx, plan_n_keep, plan_workspace : as for sparse_attn_plan.
 *   fwd_workspace : as for sparse_attn_forward, then consumed by sparse_attn_attend.
 * Same argument checks and error codes as the two calls; nothing is enqueued on error. */
int sparse_attn_plan_prepare(const sa_tensor* q, const sa_tensor* k, const sa_tensor* v,
                             int block_q, int block_k, double keep_ratio, int mode,
                             int32_t* plan_idx, int64_t plan_n_keep,
                             void* plan_workspace, size_t plan_workspace_bytes,
                             void* fwd_workspace, size_t fwd_workspace_bytes, hipStream_t stream);

/* ---- the Q/K prologue fused into the same pass ------------------------------------
 * Page "600倍加速，720p视频实时生成！单卡也能带的动14B模型", efficient inference operators
 * paragraph, and page "Run Wan2.2-A14B on One RTX 5090: 720p Video in 3.8s", section 4: 3-D RoPE
 * and RMSNorm run as fused kernels. The pages define neither; the readings, from the published
 * definitions, applied to Q and to K (not V) before the block means and the quantization:
 *   RMSNorm (Zhang and Sennrich 2019) over the D channels of each head's row:
 *     y = x / sqrt(mean(x^2) + eps) * gain[h][c];
 *   3-D RoPE (the RoFormer rotation, Su et al. 2021, of adjacent channel pairs (2p, 2p+1)):
 *     the 64 pairs split 22 / 21 / 21 over the token's grid coordinates (t, y, x) (row-major
 *     token order n = (t*grid_h + y)*grid_w + x); pair j of an axis group of m pairs turns by
 *     a = coord * theta^(-j/m): (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a).
 *   Precision: the result decides the INT8/FP8 codes, so it is computed in fp32, each IEEE
 *   operation rounded on its own: the mean square is the exact sum of the squares divided by D
 *   and rounded to fp32 (eps is rounded to fp32), r = 1 / sqrt(ms + eps), y = (x * r) * gain;
 *   cos and sin are taken in fp64 and rounded to fp32 (a table in the plan workspace, computed
 *   on the stream by the call), and the rotation's products and sums are fp32 operations with
 *   no fused multiply-add. These fp32 values are what the block means (fp64 sums) and the
 *   quantizer see. */
typedef struct sa_qk_prologue {
  const float* q_gain;  /* device fp32 [H][D], RMSNorm gain of Q, 16-byte aligned */
  const float* k_gain;  /* device fp32 [H][D], RMSNorm gain of K, 16-byte aligned */
  double eps;           /* > 0 */
  int64_t grid_t, grid_h, grid_w;  /* token grid; grid_t * grid_h * grid_w must equal L */
  double theta;         /* rotary base, > 1 (10000 in RoFormer) */
} sa_qk_prologue;

/* sparse_attn_plan without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops, harnesses that forbid hipMalloc).
 * Same arguments, checks, kernels and result as sparse_attn_plan; the scratch (block means
 * and pooled scores, sa_plan_workspace_bytes of it) is a fixed SA_PLAN_NOALLOC_MAX_BYTES
 * device array that the library holds on each GPU it runs on until the process ends.
 * Shapes needing more return SA_ERR_WORKSPACE before anything is enqueued (64 MiB covers,
 * for example, up to 8 heads of a 75600-token sequence with block_q 128, block_k 64).
 * Allocates, frees and synchronises nothing. Calls on one GPU share its array: two calls
 * whose kernels overlap on that GPU (different streams, or host threads, without ordering
 * between them) race and may both return wrong plans; order them, or use sparse_attn_plan.
 * The first call on a device looks the array's address up (hipGetSymbolAddress) with that
 * device current; SA_ERR_HIP if that fails. Returns the size limit: */
size_t sa_plan_noalloc_max_bytes(void);
int sparse_attn_plan_noalloc(const sa_tensor* q, const sa_tensor* k, int block_q, int block_k,
                             double keep_ratio, int32_t* plan_idx, int64_t plan_n_keep,
                             hipStream_t stream);

/* Plan workspace for sparse_attn_plan_prepare_prologue: sa_plan_workspace_bytes plus the
 * rotary table (8 bytes per (axis coordinate, pair)). */
int sa_plan_prologue_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t D, int block_q,
                                     int block_k, int64_t grid_t, int64_t grid_h, int64_t grid_w,
                                     size_t* bytes);

/* sparse_attn_plan_prepare with the prologue applied to Q and K first, in the same pass: the
 * plan is taken from the block means of the normalized, rotated Q and K, and the workspace
 * holds their quantized blocks (V as before), ready for sparse_attn_attend. q and k are the
 * raw (pre-norm, pre-rotation) projections, bf16. In SA_MODE_BF16 the normalized, rotated
 * values are rounded to bf16 (RNE): K into the K tiles, Q into the workspace's Q region, which
 * sparse_attn_attend then reads instead of its q argument (q still gives the shape; a later
 * sparse_attn_prepare on the workspace switches back to q). plan_workspace must hold
 * sa_plan_prologue_workspace_bytes(...) bytes. L must be below 2^31. Same conventions and
 * errors as sparse_attn_plan_prepare, plus SA_ERR_INVALID_ARG for a null gain, eps <= 0 or
 * theta <= 1 and SA_ERR_SHAPE_MISMATCH when the grid does not hold L tokens. */
int sparse_attn_plan_prepare_prologue(const sa_tensor* q, const sa_tensor* k, const sa_tensor* v,
                                      int block_q, int block_k, double keep_ratio, int mode,
                                      const sa_qk_prologue* prologue, int32_t* plan_idx,
                                      int64_t plan_n_keep, void* plan_workspace,
                                      size_t plan_workspace_bytes, void* fwd_workspace,
                                      size_t fwd_workspace_bytes, hipStream_t stream);

/* ---- the same stages one by one (per-stage timing and parity) ------------ */

/* Block means of x over blocks of `block` tokens: means fp64 [B][H][n][D], contiguous. */
int sparse_attn_pool(const sa_tensor* x, int block, double* means, hipStream_t stream);

/* Pooled scores and per-row top-n_keep of fp64 means (as written by sparse_attn_pool).
 * workspace >= 8*B*H*nQ*nK bytes (the score matrix). */
int sparse_attn_select(const double* q_means, const double* k_means, int64_t B, int64_t H,
                       int64_t nQ, int64_t nK, int64_t D, int64_t n_keep, int32_t* plan_idx,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The prepare half of sparse_attn_forward (quantize in INT8/FP8 mode). */
int sparse_attn_prepare(const sa_tensor* q, const sa_tensor* k, const sa_tensor* v,
                        int block_q, int block_k, int mode,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The attend half of sparse_attn_forward; the workspace must hold what
 * sparse_attn_prepare (or a plan_prepare call) wrote for the same q, k, v, block sizes and
 * mode. BF16 mode after sparse_attn_plan_prepare_prologue: Q is read from the workspace. */
int sparse_attn_attend(const sa_tensor* q, const int32_t* plan_idx, int block_q, int block_k,
                       int64_t n_keep, int mode, float sm_scale, const sa_tensor* out,
                       const void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- Light-Ulysses FP8 exchange payload (sequence parallelism over P peers) ------
 * Page "600倍加速，720p视频实时生成！单卡也能带的动14B模型", multi-card path, Light-Ulysses
 * paragraph; page "Run Wan2.2-A14B on One RTX 5090: 720p Video in 3.8s", section 4: tokens are
 * split over P GPUs; an all-to-all moves Q, K, V from the token split to a head split before
 * attention and the output back after it, in FP8, with Q, K and V in one payload built by fused
 * pre/post kernels, pipelined by groups of heads. These calls are the pack and unpack kernels on
 * either side of that all-to-all; the collective itself (an equal-split all-to-all of the
 * payload's P chunks) is the caller's.
 * Readings (the pages give no format):
 *   - tokens in P contiguous shards of Lmax = ceil(L/P) tokens (the last one shorter; every peer
 *     must hold at least one token), heads in P contiguous groups of H/P (H divisible by P);
 *   - every row of D = 128 values (one token, head and tensor) travels as FP8 E4M3 codes (RNE)
 *     with one power-of-two scale 2^e, e the smallest integer with max|row| <= 448 * 2^e,
 *     clamped to [-127, 127] (0 for a zero row), sent as the byte 127 + e; the receiver
 *     writes code * 2^e rounded to bf16 (exact unless below bf16's smallest subnormal);
 *   - a head chunk [head_begin, head_begin + head_count) of every group is one payload, so the
 *     exchange can run chunk by chunk (head_count = H/P moves all heads at once).
 * Payload (device memory, caller-owned, 16-byte aligned): P chunks of chunk_bytes each, chunk c
 * for peer c (destination when packing, source when unpacking): FP8 codes
 * [B][Lmax][head_count][T][128], then one scale byte per row [B][Lmax][head_count][T], then
 * padding to a multiple of 256 bytes (unspecified). Rows past the end of a short shard are sent
 * as code 0 with scale byte 127 and are not written on unpacking. T = n_tensors (1 to 3; Q, K, V
 * in the order given). Tensors are bf16 descriptors as above (any strides, D contiguous). */

/* Bytes of one chunk and of the whole payload (P chunks) for n_tensors tensors of B batches,
 * head_count heads per chunk, L tokens in total. No GPU work. */
int sa_ulysses_payload_bytes(int64_t B, int64_t head_count, int64_t L, int64_t D, int peers,
                             int n_tensors, size_t* chunk_bytes, size_t* total_bytes);

/* Token side -> payload (before attention). x: n_tensors descriptors of the local shard,
 * [B, H, L_r, D], L_r = the token count of shard `rank` of L. Chunk c receives heads
 * c*(H/P) + [head_begin, head_begin + head_count) of every token of the shard. */
int sa_ulysses_pack_seq(const sa_tensor* x, int n_tensors, int64_t L, int peers, int rank,
                        int head_begin, int head_count, void* payload, size_t payload_bytes,
                        hipStream_t stream);

/* Received payload -> head side: chunk c came from the peer holding token shard c. y:
 * n_tensors descriptors [B, head_count, L, D] (for example a head range of the peer's
 * [B, H/P, L, D] tensors); every token of every head is written. */
int sa_ulysses_unpack_head(const void* payload, size_t payload_bytes, int peers, const sa_tensor* y,
                           int n_tensors, hipStream_t stream);

/* Head side -> payload (after attention). x: [B, head_count, L, D]; chunk c receives tokens
 * of shard c. */
int sa_ulysses_pack_head(const sa_tensor* x, int n_tensors, int peers, void* payload,
                         size_t payload_bytes, hipStream_t stream);

/* Received payload -> token side: chunk c came from the peer holding head group c. y:
 * [B, H, L_r, D] of shard `rank`; heads c*(H/P) + [head_begin, head_begin + head_count) are
 * written, the others are left as they are. */
int sa_ulysses_unpack_seq(const void* payload, size_t payload_bytes, int64_t L, int peers, int rank,
                          int head_begin, int head_count, const sa_tensor* y, int n_tensors,
                          hipStream_t stream);

/* ---- block-scaled 4-bit GEMM (NVFP4 x NVFP4) ------------------------------------------
 * Page "600倍加速，720p视频实时生成！单卡也能带的动14B模型", single-card path: the NVFP4
 * paragraph (E2M1 4-bit values, one FP8 E4M3 scale per 16 consecutive elements, one FP32 scale
 * per tensor) and the efficient-inference-operators paragraph (linear, MLP and MoE layers as
 * block-scaled GEMMs with weights and activations both NVFP4, FP32 accumulation, BF16 output,
 * column bias fused into the epilogue). Readings (the encoding rule is not given):
 *   blocks of 16 along K; tensor scale S = amax / (6 * 448) (1 for an all-zero tensor); block
 *   scale s_b = E4M3_RNE(min(amax_b / fp32(6 * S), 448)); element code
 *   q = E2M1_RNE(x * inv_b), inv_b = 1 / fp32(s_b * S) (IEEE; q = 0 where s_b = 0), E2M1 values
 *   0, 0.5, 1, 1.5, 2, 3, 4, 6 with ties to the even mantissa bit, saturating at 6; every step an
 *   fp32 IEEE operation. The element stands for q * s_b * S.
 * Storage of an NVFP4 matrix [rows][K] (K a multiple of 64): codes [rows][K/2] bytes (element 2j
 *   in the low nibble of byte j, sign in bit 3), 16-byte aligned; block scales [rows][K/16] E4M3
 *   bytes, 4-byte aligned; the tensor scale as one fp32 in device memory. */

/* Scratch for sa_nvfp4_quantize (partial maxima): a fixed 4 KB. */
int sa_nvfp4_quantize_workspace_bytes(int64_t rows, int64_t K, size_t* bytes);

/* Quantize a bf16 matrix x [rows][K] (row stride ld elements, a multiple of 8; 16-byte aligned)
 * to NVFP4: codes, scales and *tensor_scale (device fp32) as above. Three launches on the stream
 * (tensor max, tensor scale, blocks); workspace >= sa_nvfp4_quantize_workspace_bytes. */
int sa_nvfp4_quantize(const void* x, int64_t rows, int64_t K, int64_t ld, uint8_t* codes,
                      uint8_t* scales, float* tensor_scale, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Y[m][n] = S_A * S_W * sum_k (q_A[m][k] s_A[m][k/16]) (q_W[n][k] s_W[n][k/16]) + bias[n], with
 * fp32 accumulation, rounded to bf16 (RNE) and written to y [M][ldy] (8-byte aligned, ldy a
 * multiple of 4 and >= N). a_*: activations [M][K] in NVFP4; w_*: weights [N][K] in NVFP4 (each
 * output column n is the dot product with weight row n); bias: bf16 [N] or NULL. K a multiple of
 * 256, N a multiple of 8, each operand's codes below 4 GiB. Each element is dequantized exactly
 * (q * s_b has at most 6 significant bits) to fp16 and multiplied on the fp16 MFMA; products are
 * exact, sums fp32. */
int sa_nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
                  const uint8_t* w_codes, const uint8_t* w_scales, const float* w_tensor_scale,
                  const void* bias, void* y, int64_t M, int64_t N, int64_t K, int64_t ldy,
                  hipStream_t stream);

/* Debug: the int32 tile S = Q^_i K^_j^T of query block i and key block
 * j = plan_idx[b][h][i][t], through the same MFMA code as the INT8 attend kernel.
 * out: device int32 [block_q][block_k], row = query, column = key (pad entries 0). */
int sparse_attn_debug_qk_tile(const void* workspace, size_t workspace_bytes,
                              int64_t B, int64_t H, int64_t L, int64_t D,
                              int block_q, int block_k, const int32_t* plan_idx, int64_t n_keep,
                              int64_t b, int64_t h, int64_t i, int64_t t,
                              int32_t* out, hipStream_t stream);

/* Debug, all-FP8 mode: the fp32 scores S = (s_q,i Q^_i)(s_k,j K^_j)^T of query block i and key
 * block j = plan_idx[b][h][i][t] from a workspace that sparse_attn_prepare filled in
 * SA_MODE_FP8, through the same scaled FP8 MFMA code as that mode's attend kernel (both
 * power-of-two block scales applied by the MFMA). The instruction sums each group of 64
 * products in its own fixed-point alignment, so S can differ from the exact sum (by about
 * 2^-12 of the group's largest product); this call lets a test measure that.
 * out: device fp32 [block_q][block_k], row = query, column = key (pad entries 0).
 * Errors: as sparse_attn_debug_qk_tile. */
int sparse_attn_debug_qk_tile_fp8(const void* workspace, size_t workspace_bytes,
                                  int64_t B, int64_t H, int64_t L, int64_t D,
                                  int block_q, int block_k, const int32_t* plan_idx, int64_t n_keep,
                                  int64_t b, int64_t h, int64_t i, int64_t t,
                                  float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
