// The output head: a causal 3x3x3 conv to a few channels (the page's conv_out), re-expressed so
// the matrix cores are not wasted on a 3-wide output. Following the kernel README's output-head
// design, the nine spatial taps become output channels of a temporal (3,1,1) conv,
//   Z[j*3+k][t, h', w'][o] = sum_{c, i} W[o, c, i, j, k] * x[c, t+i-2, h', w'],
// computed at every position by the implicit-GEMM kernel (36 outputs: 9 taps x 4 colour slots,
// fp32, one float4 per tap plane and position), and a 9-tap stencil then sums the shifted planes:
//   y[o, t, h, w] = b[o] + sum_{j,k} Z[j*3+k][t, h+j-1, w+k-1][o]   (zero outside the frame),
// which is the 3x3x3 conv with zero padding exactly (in real arithmetic).
#include "common.h"

namespace wvd {

namespace {

__device__ __forceinline__ float head_w(const void* w, int bf, int64_t i) {
  return bf ? bf16_to_f32(((const bf16_t*)w)[i]) : ((const float*)w)[i];
}

// [Npad][3][Cip]: row n = (j*3+k)*4 + o holds W[o][c][i][j][k] at [n][i][c] (zero for o >= Co).
__global__ void pack_head_kernel(const void* __restrict__ w, int w_bf16, int Co, int Ci, int Npad, int Cip,
                                 bf16_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)Npad * 3 * Cip;
  if (idx >= total) return;
  const int c = (int)(idx % Cip);
  const int i = (int)((idx / Cip) % 3);
  const int n = (int)(idx / ((int64_t)Cip * 3));
  const int o = n & 3, tap = n >> 2;
  float v = 0.0f;
  if (tap < 9 && o < Co && c < Ci) {
    const int j = tap / 3, k = tap % 3;
    v = head_w(w, w_bf16, ((((int64_t)o * Ci + c) * 3 + i) * 3 + j) * 3 + k);
  }
  out[idx] = (bf16_t)f32_to_bf16(v);
}

// One thread per output pixel: nine 16-byte tap reads (consecutive threads read consecutive
// positions of a plane: coalesced), fp32 sums in (j, k) order, one rounding per output.
__global__ __launch_bounds__(256) void head_stencil_kernel(const float4* __restrict__ Z, int Co,
                                                           const float* __restrict__ bias, bf16_t* __restrict__ video,
                                                           int64_t frames, int fbase, int T, int H, int W) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t HW = (int64_t)H * W;
  const int64_t plane = (int64_t)T * HW;
  if (idx >= plane) return;
  const int t = (int)(idx / HW);
  const int r = (int)(idx - (int64_t)t * HW);
  const int h = r / W, w = r - (r / W) * W;
  float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int hh = h + j - 1;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int ww = w + k - 1;
      if (hh < 0 || hh >= H || ww < 0 || ww >= W) continue;
      const float4 z = Z[(int64_t)(j * 3 + k) * plane + (int64_t)t * HW + (int64_t)hh * W + ww];
      a0 += z.x;
      a1 += z.y;
      a2 += z.z;
      a3 += z.w;
    }
  }
  const int64_t pix = (int64_t)(fbase + t) * HW + r;
  const float acc[4] = {a0, a1, a2, a3};
#pragma unroll
  for (int o = 0; o < 4; ++o)
    if (o < Co) video[(int64_t)o * frames * HW + pix] = (bf16_t)f32_to_bf16(acc[o] + (bias ? bias[o] : 0.0f));
}

}  // namespace

hipError_t launch_pack_head(const void* w, int w_bf16, int Co, int Ci, int Npad, int Cip, bf16_t* out, hipStream_t s) {
  const int64_t n = (int64_t)Npad * 3 * Cip;
  hipLaunchKernelGGL(pack_head_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, w, w_bf16, Co, Ci, Npad,
                     Cip, out);
  return hipGetLastError();
}

hipError_t launch_head_stencil(const float* Z, int Co, const float* bias, bf16_t* video, int64_t frames, int fbase,
                               int T, int H, int W, hipStream_t s) {
  const int64_t n = (int64_t)T * H * W;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(head_stencil_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float4*)Z, Co,
                     bias, video, frames, fbase, T, H, W);
  return hipGetLastError();
}

}  // namespace wvd
