// Direct causal convolution in fp32 (the causal conv part of the FastVideo compare page "[perf]
// PAN2 sampling: Wan2.2 VAE decode kernel, split decode, fused DiT kernels"): one thread per
// output element, fp32 fused multiply-adds over (input channel, tap). Used for the fp32 path,
// whose sizes are small; the bf16 path runs on the matrix cores.
#include "common.h"

namespace wvd {

namespace {

struct Strides {
  int64_t c, t, h, w;
};

__global__ void conv_fp32_kernel(const float* __restrict__ x, const float* __restrict__ hist,
                                 const float* __restrict__ wt, const float* __restrict__ bias, float* __restrict__ y,
                                 int Ci, int T, int H, int W, int Th, int Co, int kt, int kh, int kw, Strides sx,
                                 Strides shs, Strides sy) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)Co * T * H * W;
  if (idx >= total) return;
  // idx enumerates (o, t, h, w) with w fastest
  int64_t r = idx;
  const int w = (int)(r % W);
  r /= W;
  const int h = (int)(r % H);
  r /= H;
  const int t = (int)(r % T);
  const int o = (int)(r / T);
  const int P = 2 * (kt / 2);
  float acc = bias ? bias[o] : 0.0f;
  for (int c = 0; c < Ci; ++c) {
    for (int i = 0; i < kt; ++i) {
      const int u = t + i - P;  // source frame; negative frames come from the history
      const float* src;
      int64_t fo;
      if (u >= 0) {
        src = x + c * sx.c;
        fo = u * sx.t;
      } else if (u >= -Th) {
        src = hist + c * shs.c;
        fo = (u + Th) * shs.t;
      } else {
        continue;
      }
      const Strides& ss = (u >= 0) ? sx : shs;
      const float* wrow = wt + (((int64_t)o * Ci + c) * kt + i) * kh * kw;
      for (int j = 0; j < kh; ++j) {
        const int hh = h + j - kh / 2;
        if (hh < 0 || hh >= H) continue;
        for (int k = 0; k < kw; ++k) {
          const int ww = w + k - kw / 2;
          if (ww < 0 || ww >= W) continue;
          acc = fmaf(wrow[j * kw + k], src[fo + hh * ss.h + ww * ss.w], acc);
        }
      }
    }
  }
  y[o * sy.c + t * sy.t + h * sy.h + w * sy.w] = acc;
}

Strides make_strides(int C, int T, int H, int W, int ncthw) {
  Strides s;
  if (ncthw) {
    s.w = 1;
    s.h = W;
    s.t = (int64_t)H * W;
    s.c = (int64_t)T * H * W;
  } else {
    s.c = 1;
    s.w = C;
    s.h = (int64_t)W * C;
    s.t = (int64_t)H * W * C;
  }
  return s;
}

}  // namespace

hipError_t launch_conv_fp32(const float* x, const float* hist, const float* w, const float* bias, float* y, int Ci,
                            int T, int H, int W, int Th, int Co, int kt, int kh, int kw, int layout_ncthw,
                            hipStream_t s) {
  const int64_t total = (int64_t)Co * T * H * W;
  if (total == 0) return hipSuccess;
  const Strides sx = make_strides(Ci, T, H, W, layout_ncthw);
  const Strides sh = make_strides(Ci, Th, H, W, layout_ncthw);
  const Strides sy = make_strides(Co, T, H, W, layout_ncthw);
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(conv_fp32_kernel, dim3((unsigned)blocks), dim3(threads), 0, s, x, hist, w, bias, y, Ci, T, H, W,
                     Th, Co, kt, kh, kw, sx, sh, sy);
  return hipGetLastError();
}

}  // namespace wvd
