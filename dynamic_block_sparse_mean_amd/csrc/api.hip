// C ABI entry points: argument validation, workspace sizing and stage sequencing.
// Every check happens before anything is enqueued; a failing call enqueues nothing.
#include <math.h>
#include <algorithm>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "sa_internal.h"

namespace sa {

static thread_local char g_err[512] = "";

int set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(SA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return SA_OK;
}

static size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

static int check_tensor(const sa_tensor* t, const char* name, bool allow_fp32) {
  if (!t) return set_error(SA_ERR_INVALID_ARG, "%s: null descriptor", name);
  if (!t->data) return set_error(SA_ERR_INVALID_ARG, "%s: null data pointer", name);
  if (t->reserved != 0) return set_error(SA_ERR_INVALID_ARG, "%s: reserved field must be 0", name);
  if (t->B < 1 || t->H < 1 || t->L < 1 || t->D < 1)
    return set_error(SA_ERR_INVALID_ARG, "%s: sizes must be positive (B=%lld H=%lld L=%lld D=%lld)",
                     name, (long long)t->B, (long long)t->H, (long long)t->L, (long long)t->D);
  if (t->D != kD) return set_error(SA_ERR_UNSUPPORTED, "%s: D=%lld, only D=128 is supported", name,
                                   (long long)t->D);
  if (t->dtype != SA_DTYPE_BF16 && !(allow_fp32 && t->dtype == SA_DTYPE_FP32))
    return set_error(SA_ERR_UNSUPPORTED, "%s: dtype %d not supported here", name, t->dtype);
  if (t->stride_b < 0 || t->stride_h < 0 || t->stride_l < kD)
    return set_error(SA_ERR_UNSUPPORTED, "%s: strides must be non-negative with stride_l >= D "
                     "(the D stride is 1)", name);
  // 16-byte vector loads: base and every row start must be 16-byte aligned.
  const int64_t per16 = t->dtype == SA_DTYPE_BF16 ? 8 : 4;
  if (((uintptr_t)t->data & 15) || (t->stride_b % per16) || (t->stride_h % per16) ||
      (t->stride_l % per16))
    return set_error(SA_ERR_UNSUPPORTED, "%s: data and strides must be 16-byte aligned", name);
  return SA_OK;
}

static int same_shape(const sa_tensor* a, const sa_tensor* b, const char* an, const char* bn) {
  if (a->B != b->B || a->H != b->H || a->L != b->L || a->D != b->D)
    return set_error(SA_ERR_SHAPE_MISMATCH, "%s and %s have different shapes", an, bn);
  return SA_OK;
}

static int check_blocks(int bq, int bk) {
  if (bq != 64 && bq != 128) return set_error(SA_ERR_UNSUPPORTED, "block_q=%d not in {64,128}", bq);
  if (bk != 64 && bk != 128) return set_error(SA_ERR_UNSUPPORTED, "block_k=%d not in {64,128}", bk);
  return SA_OK;
}

// Launch limits of the path, checked before anything is enqueued: the score kernel puts the
// (batch, head) index on grid z (at most 65535), and the largest 1-D grid, the quantization
// pass, has B*H*(nQ + 2 nK) workgroups of 256 threads, whose work-item count must stay below
// 2^32 (every other grid of the path is smaller), so workgroup ids stay below 2^24, the range
// the kernels' multiply-shift id split relies on. B, H >= 1 and nQ, nK >= 0; each factor is
// bounded before the products, so nothing overflows.
static int check_grid(int64_t B, int64_t H, int64_t nQ, int64_t nK) {
  constexpr int64_t kMaxGroups = 0xFFFFFFFFLL / 256;
  const int64_t blocks = nQ + 2 * nK;
  if (B > 65535 || H > 65535 || B * H > 65535 || blocks > kMaxGroups || B * H * blocks > kMaxGroups)
    return set_error(SA_ERR_UNSUPPORTED,
                     "B=%lld H=%lld with %lld query and %lld key blocks is too large for one launch "
                     "(B*H <= 65535 and B*H*(nQ + 2 nK) <= %lld)",
                     (long long)B, (long long)H, (long long)nQ, (long long)nK, (long long)kMaxGroups);
  return SA_OK;
}

static TensorView view(const sa_tensor* t) {
  return TensorView{t->data, t->dtype, t->stride_b, t->stride_h, t->stride_l};
}

static int forward_layout(int64_t B, int64_t H, int64_t L, int64_t D, int bq, int bk, int mode,
                          sa_forward_layout* lay) {
  if (B < 1 || H < 1 || L < 1) return set_error(SA_ERR_INVALID_ARG, "sizes must be positive");
  if (D != kD) return set_error(SA_ERR_UNSUPPORTED, "D=%lld, only D=128 is supported", (long long)D);
  int st = check_blocks(bq, bk);
  if (st) return st;
  if (mode != SA_MODE_BF16 && mode != SA_MODE_INT8_FP8 && mode != SA_MODE_FP8)
    return set_error(SA_ERR_UNSUPPORTED, "mode %d unknown", mode);
  const bool quantized = mode != SA_MODE_BF16;
  const int64_t nQ = (L + bq - 1) / bq, nK = (L + bk - 1) / bk;
  if (nK > kMaxKeyBlocks)
    return set_error(SA_ERR_UNSUPPORTED, "nK=%lld key blocks exceeds %d", (long long)nK, kMaxKeyBlocks);
  if ((st = check_grid(B, H, nQ, nK))) return st;
  const int64_t BH = B * H;
  const size_t esz = quantized ? 1 : 2;
  memset(lay, 0, sizeof(*lay));
  lay->nQ = nQ;
  lay->nK = nK;
  size_t off = 0;
  // Q^ codes (quantized modes) or the prologue's bf16 Q (bf16 mode)
  lay->q_off = off;
  off = align_up(off + (size_t)BH * nQ * bq * D * esz);
  lay->k_off = off;
  off = align_up(off + (size_t)BH * nK * bk * D * esz);
  lay->v_off = off;
  off = align_up(off + (size_t)BH * nK * bk * D * esz);
  lay->sq_off = off;
  if (quantized) {
    off = align_up(off + (size_t)BH * nQ * 4);
    lay->sk_off = off;
    off = align_up(off + (size_t)BH * nK * 4);
    lay->sv_off = off;
    off = align_up(off + (size_t)BH * nK * 4);
  } else {
    off = align_up(off + 4);  // bf16 mode: the Q-source word
  }
  lay->total = off;
  return SA_OK;
}

// ---- Light-Ulysses exchange geometry ----------------------------------------------
struct UlyssesGeom {
  int64_t lmax;   // tokens per shard (the last shard may be shorter)
  int64_t rows;   // payload rows per chunk
  int64_t chunk;  // bytes per chunk, a multiple of 256
};

static int ulysses_geom(int64_t B, int64_t hc, int64_t L, int peers, int T, UlyssesGeom* g) {
  if (peers < 1 || peers > 4096) return set_error(SA_ERR_INVALID_ARG, "peers=%d not in [1, 4096]", peers);
  if (T < 1 || T > 3) return set_error(SA_ERR_INVALID_ARG, "n_tensors=%d not in [1, 3]", T);
  if (B < 1 || hc < 1 || L < 1) return set_error(SA_ERR_INVALID_ARG, "sizes must be positive");
  g->lmax = (L + peers - 1) / peers;
  if ((int64_t)(peers - 1) * g->lmax >= L)
    return set_error(SA_ERR_UNSUPPORTED, "L=%lld over %d peers leaves a peer without tokens", (long long)L, peers);
  if (g->lmax * hc * T >= ((int64_t)1 << 31) || (int64_t)peers * B > 65535)
    return set_error(SA_ERR_UNSUPPORTED, "payload too large for one launch (Lmax*head_count*T < 2^31, "
                     "peers*B <= 65535)");
  g->rows = B * g->lmax * hc * T;
  g->chunk = (int64_t)align_up((size_t)g->rows * (kD + 1));
  return SA_OK;
}

// n_tensors (1 to 3) descriptors of one shape, bf16.
static int check_ulysses_tensors(const sa_tensor* x, int T, const char* name) {
  if (!x) return set_error(SA_ERR_INVALID_ARG, "%s: null descriptor array", name);
  if (T < 1 || T > 3) return set_error(SA_ERR_INVALID_ARG, "n_tensors=%d not in [1, 3]", T);
  int st;
  for (int i = 0; i < T; ++i) {
    if ((st = check_tensor(&x[i], name, false))) return st;
    if ((st = same_shape(&x[0], &x[i], name, name))) return st;
  }
  return SA_OK;
}

static int check_payload(const void* payload, size_t bytes, int peers, const UlyssesGeom& g) {
  if (!payload) return set_error(SA_ERR_INVALID_ARG, "payload is null");
  if ((uintptr_t)payload & 15) return set_error(SA_ERR_UNSUPPORTED, "payload must be 16-byte aligned");
  const size_t need = (size_t)peers * (size_t)g.chunk;
  if (bytes < need) return set_error(SA_ERR_WORKSPACE, "payload needs %zu bytes, got %zu", need, bytes);
  return SA_OK;
}

static int check_head_chunk(int64_t H, int peers, int head_begin, int head_count) {
  if (H % peers) return set_error(SA_ERR_UNSUPPORTED, "H=%lld is not a multiple of peers=%d", (long long)H, peers);
  const int64_t group = H / peers;
  if (head_begin < 0 || head_count < 1 || head_begin + (int64_t)head_count > group)
    return set_error(SA_ERR_INVALID_ARG, "head chunk [%d, %d) not inside a group of %lld heads", head_begin,
                     head_begin + head_count, (long long)group);
  return SA_OK;
}

static int ulysses_seq_side(bool pack, const sa_tensor* x, int T, int64_t L, int peers, int rank, int head_begin,
                            int head_count, void* payload, size_t payload_bytes, hipStream_t stream) {
  int st;
  if ((st = check_ulysses_tensors(x, T, pack ? "x" : "y"))) return st;
  UlyssesGeom g;
  if ((st = ulysses_geom(x->B, head_count, L, peers, T, &g))) return st;
  if (rank < 0 || rank >= peers) return set_error(SA_ERR_INVALID_ARG, "rank=%d not in [0, %d)", rank, peers);
  if ((st = check_head_chunk(x->H, peers, head_begin, head_count))) return st;
  const int64_t shard = std::min(g.lmax, L - (int64_t)rank * g.lmax);
  if (x->L != shard)
    return set_error(SA_ERR_SHAPE_MISMATCH, "rank %d holds %lld tokens of L=%lld, the tensors have %lld", rank,
                     (long long)shard, (long long)L, (long long)x->L);
  if ((st = check_payload(payload, payload_bytes, peers, g))) return st;
  TensorView v[3];
  for (int i = 0; i < T; ++i) v[i] = view(&x[i]);
  launch_ulysses(pack, v, T, false, x->B, g.lmax, head_count, x->H / peers, head_begin, shard, peers, g.chunk,
                 (uint8_t*)payload, stream);
  return check_launch(pack ? "ulysses pack (sequence side)" : "ulysses unpack (sequence side)");
}

static int ulysses_head_side(bool pack, const sa_tensor* x, int T, int peers, void* payload, size_t payload_bytes,
                             hipStream_t stream) {
  int st;
  if ((st = check_ulysses_tensors(x, T, pack ? "x" : "y"))) return st;
  UlyssesGeom g;
  if ((st = ulysses_geom(x->B, x->H, x->L, peers, T, &g))) return st;
  if ((st = check_payload(payload, payload_bytes, peers, g))) return st;
  TensorView v[3];
  for (int i = 0; i < T; ++i) v[i] = view(&x[i]);
  launch_ulysses(pack, v, T, true, x->B, g.lmax, x->H, x->H, 0, x->L, peers, g.chunk, (uint8_t*)payload, stream);
  return check_launch(pack ? "ulysses pack (head side)" : "ulysses unpack (head side)");
}

static float log2_scale(float sm_scale, int64_t D) {
  const double sm = sm_scale > 0.f ? (double)sm_scale : 1.0 / sqrt((double)D);
  return (float)(sm * 1.4426950408889634);  // sm * log2(e), rounded once to fp32
}

}  // namespace sa

using namespace sa;

extern "C" {

const char* sa_status_string(int status) {
  switch (status) {
    case SA_OK: return "ok";
    case SA_ERR_INVALID_ARG: return "invalid argument";
    case SA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SA_ERR_WORKSPACE: return "workspace missing or too small";
    case SA_ERR_SHAPE_MISMATCH: return "shape mismatch";
    case SA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* sa_last_error(void) { return g_err; }

int64_t sa_num_blocks(int64_t L, int64_t block) {
  if (L < 1 || block < 1) return -1;
  return (L + block - 1) / block;
}

int64_t sa_plan_n_keep(int64_t nK, double keep_ratio) {
  if (nK < 1 || !(keep_ratio > 0.0) || keep_ratio > 1.0) return -1;
  int64_t n = (int64_t)ceil(keep_ratio * (double)nK - 1e-6);
  if (n < 1) n = 1;
  if (n > nK) n = nK;
  return n;
}

int sa_plan_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t D, int block_q, int block_k,
                            size_t* bytes) {
  if (!bytes) return set_error(SA_ERR_INVALID_ARG, "bytes is null");
  if (B < 1 || H < 1 || L < 1) return set_error(SA_ERR_INVALID_ARG, "sizes must be positive");
  if (D != kD) return set_error(SA_ERR_UNSUPPORTED, "only D=128 is supported");
  int st = check_blocks(block_q, block_k);
  if (st) return st;
  const int64_t nQ = (L + block_q - 1) / block_q, nK = (L + block_k - 1) / block_k;
  if (nK > kMaxKeyBlocks) return set_error(SA_ERR_UNSUPPORTED, "too many key blocks");
  if ((st = check_grid(B, H, nQ, nK))) return st;
  const int64_t BH = B * H;
  *bytes = align_up((size_t)BH * nQ * D * 8) + align_up((size_t)BH * nK * D * 8) +
           align_up((size_t)BH * nQ * nK * 8);
  return SA_OK;
}

int sa_forward_workspace_layout(int64_t B, int64_t H, int64_t L, int64_t D, int block_q,
                                int block_k, int mode, sa_forward_layout* layout) {
  if (!layout) return set_error(SA_ERR_INVALID_ARG, "layout is null");
  return forward_layout(B, H, L, D, block_q, block_k, mode, layout);
}

int sa_forward_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t D, int block_q,
                               int block_k, int mode, size_t* bytes) {
  if (!bytes) return set_error(SA_ERR_INVALID_ARG, "bytes is null");
  sa_forward_layout lay;
  int st = forward_layout(B, H, L, D, block_q, block_k, mode, &lay);
  if (st) return st;
  *bytes = lay.total;
  return SA_OK;
}

int sparse_attn_pool(const sa_tensor* x, int block, double* means, hipStream_t stream) {
  int st = check_tensor(x, "x", true);
  if (st) return st;
  if (block != 64 && block != 128) return set_error(SA_ERR_UNSUPPORTED, "block=%d not in {64,128}", block);
  if (!means) return set_error(SA_ERR_INVALID_ARG, "means is null");
  if ((st = check_grid(x->B, x->H, (x->L + block - 1) / block, 0))) return st;
  launch_pool(view(x), x->B, x->H, x->L, block, means, stream);
  return check_launch("pool");
}

static int select_checked(const double* qm, const double* km, int64_t B, int64_t H, int64_t nQ,
                          int64_t nK, int64_t n_keep, int32_t* plan, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  const size_t need = (size_t)B * H * nQ * nK * 8;
  if (!ws || ws_bytes < need)
    return set_error(SA_ERR_WORKSPACE, "select needs %zu workspace bytes, got %zu", need, ws_bytes);
  launch_scores(qm, km, B * H, nQ, nK, (double*)ws, stream);
  int st = check_launch("scores");
  if (st) return st;
  launch_topk((const double*)ws, B * H * nQ, nK, n_keep, plan, stream);
  return check_launch("topk");
}

int sparse_attn_select(const double* q_means, const double* k_means, int64_t B, int64_t H,
                       int64_t nQ, int64_t nK, int64_t D, int64_t n_keep, int32_t* plan_idx,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q_means || !k_means || !plan_idx) return set_error(SA_ERR_INVALID_ARG, "null pointer");
  if (B < 1 || H < 1 || nQ < 1 || nK < 1) return set_error(SA_ERR_INVALID_ARG, "sizes must be positive");
  if (D != kD) return set_error(SA_ERR_UNSUPPORTED, "only D=128 is supported");
  if (nK > kMaxKeyBlocks) return set_error(SA_ERR_UNSUPPORTED, "nK exceeds %d", kMaxKeyBlocks);
  if (n_keep < 1 || n_keep > nK) return set_error(SA_ERR_INVALID_ARG, "n_keep=%lld not in [1, nK]",
                                                  (long long)n_keep);
  const int st = check_grid(B, H, nQ, nK);
  if (st) return st;
  return select_checked(q_means, k_means, B, H, nQ, nK, n_keep, plan_idx, workspace,
                        workspace_bytes, stream);
}

// Argument checks of sparse_attn_plan; on success *n_keep, *nQ, *nK are set.
static int plan_args(const sa_tensor* q, const sa_tensor* k, int block_q, int block_k, double keep_ratio,
                     const int32_t* plan_idx, int64_t plan_n_keep, size_t workspace_bytes, const void* workspace,
                     int64_t* n_keep, int64_t* nQ, int64_t* nK) {
  int st = check_tensor(q, "q", true);
  if (st) return st;
  if ((st = check_tensor(k, "k", true))) return st;
  if ((st = same_shape(q, k, "q", "k"))) return st;
  if ((st = check_blocks(block_q, block_k))) return st;
  if (!plan_idx) return set_error(SA_ERR_INVALID_ARG, "plan_idx is null");
  *nQ = (q->L + block_q - 1) / block_q;
  *nK = (q->L + block_k - 1) / block_k;
  if (*nK > kMaxKeyBlocks) return set_error(SA_ERR_UNSUPPORTED, "nK exceeds %d", kMaxKeyBlocks);
  *n_keep = sa_plan_n_keep(*nK, keep_ratio);
  if (*n_keep < 0) return set_error(SA_ERR_INVALID_ARG, "keep_ratio=%g not in (0, 1]", keep_ratio);
  if (plan_n_keep != *n_keep)
    return set_error(SA_ERR_SHAPE_MISMATCH, "plan row length %lld, keep_ratio gives %lld",
                     (long long)plan_n_keep, (long long)*n_keep);
  size_t need = 0;
  if ((st = sa_plan_workspace_bytes(q->B, q->H, q->L, q->D, block_q, block_k, &need))) return st;
  if (!workspace || workspace_bytes < need)
    return set_error(SA_ERR_WORKSPACE, "plan needs %zu workspace bytes, got %zu", need, workspace_bytes);
  return SA_OK;
}

static int prepare_checked(const sa_tensor* q, const sa_tensor* k, const sa_tensor* v, int bq,
                           int bk, int mode, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_tensor(q, "q", false);
  if (st) return st;
  if ((st = check_tensor(k, "k", false))) return st;
  if ((st = check_tensor(v, "v", false))) return st;
  if ((st = same_shape(q, k, "q", "k")) || (st = same_shape(q, v, "q", "v"))) return st;
  sa_forward_layout lay;
  if ((st = forward_layout(q->B, q->H, q->L, q->D, bq, bk, mode, &lay))) return st;
  if (!ws || ws_bytes < lay.total)
    return set_error(SA_ERR_WORKSPACE, "forward needs %zu workspace bytes, got %zu", lay.total, ws_bytes);
  if (mode != SA_MODE_BF16) {
    launch_quant(view(q), view(k), view(v), q->B, q->H, q->L, bq, bk, lay, (char*)ws, nullptr, nullptr,
                 mode == SA_MODE_FP8, nullptr, stream);
    return check_launch("quantize");
  }
  launch_layout_bf16(view(k), view(v), q->B, q->H, q->L, bk, lay, (char*)ws, stream);
  return check_launch("layout bf16");
}

static int attend_checked(const sa_tensor* q, const int32_t* plan, int bq, int bk, int64_t n_keep,
                          int mode, float sm_scale, const sa_tensor* out, const void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  int st = check_tensor(q, "q", false);
  if (st) return st;
  if ((st = check_tensor(out, "out", false))) return st;
  if ((st = same_shape(q, out, "q", "out"))) return st;
  if (!plan) return set_error(SA_ERR_INVALID_ARG, "plan_idx is null");
  sa_forward_layout lay;
  if ((st = forward_layout(q->B, q->H, q->L, q->D, bq, bk, mode, &lay))) return st;
  if (n_keep < 1 || n_keep > lay.nK)
    return set_error(SA_ERR_INVALID_ARG, "n_keep=%lld not in [1, nK=%lld]", (long long)n_keep,
                     (long long)lay.nK);
  if (!ws || ws_bytes < lay.total)
    return set_error(SA_ERR_WORKSPACE, "forward needs %zu workspace bytes, got %zu", lay.total, ws_bytes);
  if (out->data == q->data) return set_error(SA_ERR_INVALID_ARG, "out aliases q");
  const float c = log2_scale(sm_scale, q->D);
  if (mode != SA_MODE_BF16) {
    launch_attend_i8f8(lay, (const char*)ws, plan, q->B, q->H, q->L, bq, bk, n_keep, c, mode == SA_MODE_FP8,
                       view(out), stream);
    return check_launch(mode == SA_MODE_FP8 ? "attend fp8" : "attend int8/fp8");
  }
  launch_attend_bf16(view(q), lay, (const char*)ws, plan, q->B, q->H, q->L, bq, bk, n_keep, c,
                     view(out), stream);
  return check_launch("attend bf16");
}

int sparse_attn_prepare(const sa_tensor* q, const sa_tensor* k, const sa_tensor* v, int block_q,
                        int block_k, int mode, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  return prepare_checked(q, k, v, block_q, block_k, mode, workspace, workspace_bytes, stream);
}

int sparse_attn_attend(const sa_tensor* q, const int32_t* plan_idx, int block_q, int block_k,
                       int64_t n_keep, int mode, float sm_scale, const sa_tensor* out,
                       const void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return attend_checked(q, plan_idx, block_q, block_k, n_keep, mode, sm_scale, out, workspace,
                        workspace_bytes, stream);
}

int sparse_attn_forward(const sa_tensor* q, const sa_tensor* k, const sa_tensor* v,
                        const int32_t* plan_idx, int block_q, int block_k, int64_t n_keep, int mode,
                        float sm_scale, const sa_tensor* out, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  // Validate everything up front so that a bad attend argument enqueues no prepare work.
  int st = check_tensor(q, "q", false);
  if (st) return st;
  if ((st = check_tensor(out, "out", false))) return st;
  if ((st = same_shape(q, out, "q", "out"))) return st;
  if (!plan_idx) return set_error(SA_ERR_INVALID_ARG, "plan_idx is null");
  if (out->data == q->data || (k && out->data == k->data) || (v && out->data == v->data))
    return set_error(SA_ERR_INVALID_ARG, "out aliases an input");
  const int64_t nK = sa_num_blocks(q->L, block_k);
  if (n_keep < 1 || n_keep > nK)
    return set_error(SA_ERR_INVALID_ARG, "n_keep=%lld not in [1, nK=%lld]", (long long)n_keep,
                     (long long)nK);
  if ((st = prepare_checked(q, k, v, block_q, block_k, mode, workspace, workspace_bytes, stream)))
    return st;
  return attend_checked(q, plan_idx, block_q, block_k, n_keep, mode, sm_scale, out, workspace,
                        workspace_bytes, stream);
}

// Plan workspace pieces: Q means, K means, score matrix.
static void plan_pieces(const sa_tensor* q, int64_t nQ, int64_t nK, void* workspace, double** qm,
                        double** km, char** scores) {
  const int64_t BH = q->B * q->H;
  char* ws = (char*)workspace;
  *qm = (double*)ws;
  *km = (double*)(ws + align_up((size_t)BH * nQ * kD * 8));
  *scores = ws + align_up((size_t)BH * nQ * kD * 8) + align_up((size_t)BH * nK * kD * 8);
}

int sparse_attn_plan(const sa_tensor* q, const sa_tensor* k, int block_q, int block_k,
                     double keep_ratio, int32_t* plan_idx, int64_t plan_n_keep, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  int64_t n_keep, nQ, nK;
  int st = plan_args(q, k, block_q, block_k, keep_ratio, plan_idx, plan_n_keep, workspace_bytes, workspace,
                     &n_keep, &nQ, &nK);
  if (st) return st;
  double *qm, *km;
  char* scores;
  plan_pieces(q, nQ, nK, workspace, &qm, &km, &scores);
  launch_pool(view(q), q->B, q->H, q->L, block_q, qm, stream);
  if ((st = check_launch("pool q"))) return st;
  launch_pool(view(k), k->B, k->H, k->L, block_k, km, stream);
  if ((st = check_launch("pool k"))) return st;
  return select_checked(qm, km, q->B, q->H, nQ, nK, n_keep, plan_idx, scores,
                        (size_t)q->B * q->H * nQ * nK * 8, stream);
}

// ---- the plan without a caller workspace ------------------------------------------------
// The plan's scratch (block means and the pooled score matrix) in a file-scope device array:
// each GPU the library runs on holds one copy for the life of the process. Host code never
// passes the array's name to a kernel or a copy (on the host it only stands in for the
// symbol); it uses the device address hipGetSymbolAddress returns, fetched once per device
// with that device current.
static __device__ __align__(256) unsigned char scratch[SA_PLAN_NOALLOC_MAX_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_error(SA_ERR_HIP, "no current HIP device (or device id %d beyond %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(SA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SA_OK;
}

size_t sa_plan_noalloc_max_bytes(void) { return (size_t)SA_PLAN_NOALLOC_MAX_BYTES; }

int sparse_attn_plan_noalloc(const sa_tensor* q, const sa_tensor* k, int block_q, int block_k,
                             double keep_ratio, int32_t* plan_idx, int64_t plan_n_keep, hipStream_t stream) {
  // every argument check of sparse_attn_plan first (a dummy workspace pointer of the maximum
  // size stands in for the scratch), so nothing touches the device on a bad call
  int64_t n_keep, nQ, nK;
  int st = plan_args(q, k, block_q, block_k, keep_ratio, plan_idx, plan_n_keep, ~(size_t)0,
                     (const void*)plan_idx, &n_keep, &nQ, &nK);
  if (st) return st;
  size_t need = 0;
  if ((st = sa_plan_workspace_bytes(q->B, q->H, q->L, q->D, block_q, block_k, &need))) return st;
  if (need > (size_t)SA_PLAN_NOALLOC_MAX_BYTES)
    return set_error(SA_ERR_WORKSPACE,
                     "sparse_attn_plan_noalloc: this shape needs %zu scratch bytes, above its fixed %zu "
                     "(use sparse_attn_plan with a workspace)", need, (size_t)SA_PLAN_NOALLOC_MAX_BYTES);
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  // pool and select overwrite every byte they read back, so the scratch needs no clearing
  return sparse_attn_plan(q, k, block_q, block_k, keep_ratio, plan_idx, plan_n_keep, ws,
                          (size_t)SA_PLAN_NOALLOC_MAX_BYTES, stream);
}

static size_t plan_bytes(int64_t BH, int64_t nQ, int64_t nK) {
  return align_up((size_t)BH * nQ * kD * 8) + align_up((size_t)BH * nK * kD * 8) + align_up((size_t)BH * nQ * nK * 8);
}

static int check_prologue(const sa_qk_prologue* pro, const sa_tensor* q) {
  if (!pro->q_gain || !pro->k_gain) return set_error(SA_ERR_INVALID_ARG, "prologue: null gain pointer");
  if (((uintptr_t)pro->q_gain & 15) || ((uintptr_t)pro->k_gain & 15))
    return set_error(SA_ERR_UNSUPPORTED, "prologue: gains must be 16-byte aligned");
  if (!((float)pro->eps > 0.f) || !isfinite((float)pro->eps))
    return set_error(SA_ERR_INVALID_ARG, "prologue: eps=%g must be positive and finite in fp32", pro->eps);
  if (!(pro->theta > 1.0) || !isfinite(pro->theta))
    return set_error(SA_ERR_INVALID_ARG, "prologue: theta=%g must be finite and > 1", pro->theta);
  if (pro->grid_t < 1 || pro->grid_h < 1 || pro->grid_w < 1)
    return set_error(SA_ERR_INVALID_ARG, "prologue: grid sizes must be positive");
  if (q->L >= ((int64_t)1 << 31) || pro->grid_t * pro->grid_h * pro->grid_w != q->L)
    return set_error(SA_ERR_SHAPE_MISMATCH, "prologue: grid %lldx%lldx%lld does not hold L=%lld tokens (< 2^31)",
                     (long long)pro->grid_t, (long long)pro->grid_h, (long long)pro->grid_w, (long long)q->L);
  return SA_OK;
}

static int plan_prepare_impl(const sa_tensor* q, const sa_tensor* k, const sa_tensor* v, int block_q,
                             int block_k, double keep_ratio, int mode, const sa_qk_prologue* pro,
                             int32_t* plan_idx, int64_t plan_n_keep, void* plan_workspace,
                             size_t plan_workspace_bytes, void* fwd_workspace, size_t fwd_workspace_bytes,
                             hipStream_t stream) {
  int64_t n_keep, nQ, nK;
  int st = plan_args(q, k, block_q, block_k, keep_ratio, plan_idx, plan_n_keep, plan_workspace_bytes,
                     plan_workspace, &n_keep, &nQ, &nK);
  if (st) return st;
  // the checks of prepare, before anything is enqueued
  if ((st = check_tensor(q, "q", false)) || (st = check_tensor(k, "k", false))) return st;
  if ((st = check_tensor(v, "v", false))) return st;
  if ((st = same_shape(q, v, "q", "v"))) return st;
  sa_forward_layout lay;
  if ((st = forward_layout(q->B, q->H, q->L, q->D, block_q, block_k, mode, &lay))) return st;
  if (!fwd_workspace || fwd_workspace_bytes < lay.total)
    return set_error(SA_ERR_WORKSPACE, "forward needs %zu workspace bytes, got %zu", lay.total,
                     fwd_workspace_bytes);
  QkPrologue qp{};
  if (pro) {
    if ((st = check_prologue(pro, q))) return st;
    const size_t base = plan_bytes(q->B * q->H, nQ, nK);
    const size_t need = base + rope_table_bytes(pro->grid_t, pro->grid_h, pro->grid_w);
    if (plan_workspace_bytes < need)
      return set_error(SA_ERR_WORKSPACE, "plan with prologue needs %zu workspace bytes, got %zu", need,
                       plan_workspace_bytes);
    qp = QkPrologue{pro->q_gain, pro->k_gain, (float)pro->eps, pro->grid_t, pro->grid_h, pro->grid_w, pro->theta,
                    (float2*)((char*)plan_workspace + base)};
  }
  double *qm, *km;
  char* scores;
  plan_pieces(q, nQ, nK, plan_workspace, &qm, &km, &scores);
  if (mode == SA_MODE_BF16) {
    if (pro) {
      launch_prologue_bf16(view(q), view(k), view(v), q->B, q->H, q->L, block_q, block_k, lay, (char*)fwd_workspace,
                           qm, km, qp, stream);
      if ((st = check_launch("prologue bf16"))) return st;
      return select_checked(qm, km, q->B, q->H, nQ, nK, n_keep, plan_idx, scores,
                            (size_t)q->B * q->H * nQ * nK * 8, stream);
    }
    if ((st = sparse_attn_plan(q, k, block_q, block_k, keep_ratio, plan_idx, plan_n_keep, plan_workspace,
                               plan_workspace_bytes, stream)))
      return st;
    return prepare_checked(q, k, v, block_q, block_k, mode, fwd_workspace, fwd_workspace_bytes, stream);
  }
  launch_quant(view(q), view(k), view(v), q->B, q->H, q->L, block_q, block_k, lay, (char*)fwd_workspace, qm,
               km, mode == SA_MODE_FP8, pro ? &qp : nullptr, stream);
  if ((st = check_launch("quantize with block means"))) return st;
  return select_checked(qm, km, q->B, q->H, nQ, nK, n_keep, plan_idx, scores,
                        (size_t)q->B * q->H * nQ * nK * 8, stream);
}

int sparse_attn_plan_prepare(const sa_tensor* q, const sa_tensor* k, const sa_tensor* v, int block_q,
                             int block_k, double keep_ratio, int mode, int32_t* plan_idx,
                             int64_t plan_n_keep, void* plan_workspace, size_t plan_workspace_bytes,
                             void* fwd_workspace, size_t fwd_workspace_bytes, hipStream_t stream) {
  return plan_prepare_impl(q, k, v, block_q, block_k, keep_ratio, mode, nullptr, plan_idx, plan_n_keep,
                           plan_workspace, plan_workspace_bytes, fwd_workspace, fwd_workspace_bytes, stream);
}

int sa_plan_prologue_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t D, int block_q, int block_k,
                                     int64_t grid_t, int64_t grid_h, int64_t grid_w, size_t* bytes) {
  int st = sa_plan_workspace_bytes(B, H, L, D, block_q, block_k, bytes);
  if (st) return st;
  if (grid_t < 1 || grid_h < 1 || grid_w < 1 || grid_t * grid_h * grid_w != L)
    return set_error(SA_ERR_SHAPE_MISMATCH, "grid %lldx%lldx%lld does not hold L=%lld tokens", (long long)grid_t,
                     (long long)grid_h, (long long)grid_w, (long long)L);
  *bytes += align_up(rope_table_bytes(grid_t, grid_h, grid_w));
  return SA_OK;
}

int sparse_attn_plan_prepare_prologue(const sa_tensor* q, const sa_tensor* k, const sa_tensor* v, int block_q,
                                      int block_k, double keep_ratio, int mode, const sa_qk_prologue* prologue,
                                      int32_t* plan_idx, int64_t plan_n_keep, void* plan_workspace,
                                      size_t plan_workspace_bytes, void* fwd_workspace, size_t fwd_workspace_bytes,
                                      hipStream_t stream) {
  if (!prologue) return set_error(SA_ERR_INVALID_ARG, "prologue is null");
  return plan_prepare_impl(q, k, v, block_q, block_k, keep_ratio, mode, prologue, plan_idx, plan_n_keep,
                           plan_workspace, plan_workspace_bytes, fwd_workspace, fwd_workspace_bytes, stream);
}

static int debug_qk_tile(const void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                         int64_t L, int64_t D, int block_q, int block_k, const int32_t* plan_idx,
                         int64_t n_keep, int64_t b, int64_t h, int64_t i, int64_t t, bool qk_fp8,
                         void* out, hipStream_t stream) {
  sa_forward_layout lay;
  int st = forward_layout(B, H, L, D, block_q, block_k, qk_fp8 ? SA_MODE_FP8 : SA_MODE_INT8_FP8, &lay);
  if (st) return st;
  if (!workspace || workspace_bytes < lay.total)
    return set_error(SA_ERR_WORKSPACE, "workspace too small");
  if (!plan_idx || !out) return set_error(SA_ERR_INVALID_ARG, "null pointer");
  if (n_keep < 1 || n_keep > lay.nK || b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= lay.nQ ||
      t < 0 || t >= n_keep)
    return set_error(SA_ERR_INVALID_ARG, "tile index out of range");
  launch_debug_qk(lay, (const char*)workspace, plan_idx, B, H, L, block_q, block_k, n_keep, b, h, i,
                  t, qk_fp8, out, stream);
  return check_launch("debug qk tile");
}

int sparse_attn_debug_qk_tile(const void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                              int64_t L, int64_t D, int block_q, int block_k,
                              const int32_t* plan_idx, int64_t n_keep, int64_t b, int64_t h,
                              int64_t i, int64_t t, int32_t* out, hipStream_t stream) {
  return debug_qk_tile(workspace, workspace_bytes, B, H, L, D, block_q, block_k, plan_idx, n_keep, b, h,
                       i, t, false, out, stream);
}

int sparse_attn_debug_qk_tile_fp8(const void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                                  int64_t L, int64_t D, int block_q, int block_k,
                                  const int32_t* plan_idx, int64_t n_keep, int64_t b, int64_t h,
                                  int64_t i, int64_t t, float* out, hipStream_t stream) {
  return debug_qk_tile(workspace, workspace_bytes, B, H, L, D, block_q, block_k, plan_idx, n_keep, b, h,
                       i, t, true, out, stream);
}

int sa_ulysses_payload_bytes(int64_t B, int64_t head_count, int64_t L, int64_t D, int peers, int n_tensors,
                             size_t* chunk_bytes, size_t* total_bytes) {
  if (!chunk_bytes || !total_bytes) return set_error(SA_ERR_INVALID_ARG, "null output pointer");
  if (D != kD) return set_error(SA_ERR_UNSUPPORTED, "D=%lld, only D=128 is supported", (long long)D);
  UlyssesGeom g;
  int st = ulysses_geom(B, head_count, L, peers, n_tensors, &g);
  if (st) return st;
  *chunk_bytes = (size_t)g.chunk;
  *total_bytes = (size_t)g.chunk * (size_t)peers;
  return SA_OK;
}

int sa_ulysses_pack_seq(const sa_tensor* x, int n_tensors, int64_t L, int peers, int rank, int head_begin,
                        int head_count, void* payload, size_t payload_bytes, hipStream_t stream) {
  return ulysses_seq_side(true, x, n_tensors, L, peers, rank, head_begin, head_count, payload, payload_bytes,
                          stream);
}

int sa_ulysses_unpack_head(const void* payload, size_t payload_bytes, int peers, const sa_tensor* y,
                           int n_tensors, hipStream_t stream) {
  return ulysses_head_side(false, y, n_tensors, peers, const_cast<void*>(payload), payload_bytes, stream);
}

int sa_ulysses_pack_head(const sa_tensor* x, int n_tensors, int peers, void* payload, size_t payload_bytes,
                         hipStream_t stream) {
  return ulysses_head_side(true, x, n_tensors, peers, payload, payload_bytes, stream);
}

int sa_ulysses_unpack_seq(const void* payload, size_t payload_bytes, int64_t L, int peers, int rank,
                          int head_begin, int head_count, const sa_tensor* y, int n_tensors, hipStream_t stream) {
  return ulysses_seq_side(false, y, n_tensors, L, peers, rank, head_begin, head_count,
                          const_cast<void*>(payload), payload_bytes, stream);
}

int sa_nvfp4_quantize_workspace_bytes(int64_t rows, int64_t K, size_t* bytes) {
  if (!bytes) return set_error(SA_ERR_INVALID_ARG, "bytes is null");
  if (rows < 1 || K < 1) return set_error(SA_ERR_INVALID_ARG, "sizes must be positive");
  *bytes = (size_t)kNvfp4Parts * sizeof(float);
  return SA_OK;
}

int sa_nvfp4_quantize(const void* x, int64_t rows, int64_t K, int64_t ld, uint8_t* codes, uint8_t* scales,
                      float* tensor_scale, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!x || !codes || !scales || !tensor_scale) return set_error(SA_ERR_INVALID_ARG, "null pointer");
  if (rows < 1 || K < 1) return set_error(SA_ERR_INVALID_ARG, "sizes must be positive");
  if (K % 64) return set_error(SA_ERR_UNSUPPORTED, "K=%lld is not a multiple of 64", (long long)K);
  if (ld < K || ld % 8) return set_error(SA_ERR_UNSUPPORTED, "ld=%lld must be >= K and a multiple of 8", (long long)ld);
  if (((uintptr_t)x & 15) || ((uintptr_t)codes & 15) || ((uintptr_t)scales & 3) || ((uintptr_t)tensor_scale & 3))
    return set_error(SA_ERR_UNSUPPORTED, "x and codes must be 16-byte aligned, scales 4-byte aligned");
  if (!workspace || workspace_bytes < (size_t)kNvfp4Parts * sizeof(float))
    return set_error(SA_ERR_WORKSPACE, "quantize needs %zu workspace bytes", (size_t)kNvfp4Parts * sizeof(float));
  const int64_t chunks = rows * (K / 8);
  const int nparts = (int)std::min<int64_t>(kNvfp4Parts, (chunks + 255) / 256);
  launch_nvfp4_quantize((const uint16_t*)x, rows, K, ld, codes, scales, tensor_scale, (float*)workspace, nparts,
                        stream);
  return check_launch("nvfp4 quantize");
}

int sa_nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
                  const uint8_t* w_codes, const uint8_t* w_scales, const float* w_tensor_scale, const void* bias,
                  void* y, int64_t M, int64_t N, int64_t K, int64_t ldy, hipStream_t stream) {
  if (!a_codes || !a_scales || !a_tensor_scale || !w_codes || !w_scales || !w_tensor_scale || !y)
    return set_error(SA_ERR_INVALID_ARG, "null pointer");
  if (M < 1 || N < 1 || K < 1) return set_error(SA_ERR_INVALID_ARG, "sizes must be positive");
  if (K % 256 || N % 8)
    return set_error(SA_ERR_UNSUPPORTED, "K=%lld must be a multiple of 256 and N=%lld of 8", (long long)K,
                     (long long)N);
  if ((M + 255) / 256 * ((N + 255) / 256) > 0x7FFFFFFFLL || N > ((int64_t)1 << 30) || K > ((int64_t)1 << 30) || M * (K / 2) > 0xFFFFFFFFLL ||
      N * (K / 2) > 0xFFFFFFFFLL)
    return set_error(SA_ERR_UNSUPPORTED, "sizes too large for one launch (each operand's codes below 4 GiB)");
  if (ldy < N || ldy % 4) return set_error(SA_ERR_UNSUPPORTED, "ldy=%lld must be >= N and a multiple of 4", (long long)ldy);
  if (((uintptr_t)a_codes & 15) || ((uintptr_t)w_codes & 15) || ((uintptr_t)a_scales & 3) ||
      ((uintptr_t)w_scales & 3) || ((uintptr_t)y & 7) || ((uintptr_t)bias & 1))
    return set_error(SA_ERR_UNSUPPORTED, "codes must be 16-byte, scales 4-byte, y 8-byte aligned");
  launch_nvfp4_gemm(a_codes, a_scales, a_tensor_scale, w_codes, w_scales, w_tensor_scale, (const uint16_t*)bias,
                    (uint16_t*)y, (int)M, (int)N, (int)K, ldy, stream);
  return check_launch("nvfp4 gemm");
}

}  // extern "C"
