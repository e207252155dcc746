// Block-mean pooling: means[bh][i][:] = mean of x[b,h,n,:] over the tokens n of block i.
//
// The importance estimate starts from block-level means of Q and K (page
// "600倍加速，720p视频实时生成！单卡也能带的动14B模型", dynamic sparse quantized attention
// paragraph; page "Run Wan2.2-A14B on One RTX 5090", section 3). A short last block is
// averaged over its own tokens. Sums are taken in fp64 (bf16 and fp32 inputs add up
// exactly or to within 2^-53), so the pooled scores and the block choice do not depend on
// summation order.
//
// HBM-bound: every element of x is read once with 16-byte streaming (nontemporal) loads; one
// workgroup of 256 threads per (batch, head, block): 16 threads cover a 128-wide row, 16 rows
// per pass.
#include "sa_internal.h"

namespace sa {

template <int BLOCK, bool BF16>
__global__ __launch_bounds__(256) void pool_kernel(const void* __restrict__ x, DivMagic H, int64_t L,
                                                   int64_t sb, int64_t sh, int64_t sl, DivMagic nb,
                                                   double* __restrict__ means) {
  constexpr int RPT = BLOCK / 16;  // rows per thread
  __shared__ double part[16][kD + 2];
  const uint32_t wg = blockIdx.x, bh32 = div_magic(wg, nb), b32 = div_magic(bh32, H);
  const int64_t nblk = nb.d, bh = bh32, blk = wg - bh32 * nb.d, b = b32, h = bh32 - b32 * H.d;
  const int t = threadIdx.x, cg = t & 15, r0 = t >> 4;
  const int64_t row0 = blk * BLOCK;
  const int count = (int)((L - row0) < BLOCK ? (L - row0) : BLOCK);
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  if (BF16) {
    const uint16_t* base = (const uint16_t*)x + b * sb + h * sh + row0 * sl + cg * 8;
    uint4 v[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int r = r0 + 16 * k;
      if (r < count) v[k] = load_stream(base + (int64_t)r * sl);
      else v[k] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += (double)__uint_as_float(w[e] << 16);
        acc[2 * e + 1] += (double)__uint_as_float(w[e] & 0xffff0000u);
      }
    }
  } else {
    const float* base = (const float*)x + b * sb + h * sh + row0 * sl + cg * 8;
    float4 v[RPT][2];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int r = r0 + 16 * k;
      if (r < count) {
        v[k][0] = *(const float4*)(base + (int64_t)r * sl);
        v[k][1] = *(const float4*)(base + (int64_t)r * sl + 4);
      } else {
        v[k][0] = v[k][1] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      acc[0] += (double)v[k][0].x; acc[1] += (double)v[k][0].y;
      acc[2] += (double)v[k][0].z; acc[3] += (double)v[k][0].w;
      acc[4] += (double)v[k][1].x; acc[5] += (double)v[k][1].y;
      acc[6] += (double)v[k][1].z; acc[7] += (double)v[k][1].w;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[r0][cg * 8 + e] = acc[e];
  __syncthreads();
  if (t < kD) {
    double s = 0.0;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += part[r][t];
    means[(bh * nblk + blk) * kD + t] = s / (double)count;
  }
}

void launch_pool(const TensorView& x, int64_t B, int64_t H, int64_t L, int block, double* means,
                 hipStream_t s) {
  const int64_t nblk = (L + block - 1) / block;
  const dim3 grid((unsigned)(B * H * nblk)), blk(256);  // below 2^24 workgroups (checked by the caller)
  const bool bf16 = x.dtype == SA_DTYPE_BF16;
  const DivMagic hd = div_magic_for((uint32_t)H), nb = div_magic_for((uint32_t)nblk);
  if (block == 64) {
    if (bf16) pool_kernel<64, true><<<grid, blk, 0, s>>>(x.data, hd, L, x.sb, x.sh, x.sl, nb, means);
    else pool_kernel<64, false><<<grid, blk, 0, s>>>(x.data, hd, L, x.sb, x.sh, x.sl, nb, means);
  } else {
    if (bf16) pool_kernel<128, true><<<grid, blk, 0, s>>>(x.data, hd, L, x.sb, x.sh, x.sl, nb, means);
    else pool_kernel<128, false><<<grid, blk, 0, s>>>(x.data, hd, L, x.sb, x.sh, x.sl, nb, means);
  }
}

}  // namespace sa
