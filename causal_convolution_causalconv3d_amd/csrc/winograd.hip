// Winograd F(2x2, 3x3) in space for the causal 3x3x3 convolution, the causal 3-tap time
// convolution kept as it is (the decoder of the FastVideo compare page "[perf] PAN2 sampling:
// Wan2.2 VAE decode kernel, split decode, fused DiT kernels" runs its up blocks' convolutions as
// Winograd products, "How the decoder got here", "The design").
//
// Each 2x2 output tile of a frame needs the 4x4 input tile d around it (rows 2ty-1 .. 2ty+2,
// columns 2tx-1 .. 2tx+2, zero outside the frame). With the F(2,3) matrices
//   B^T = [1 0 -1 0; 0 1 1 0; 0 -1 1 0; 0 1 0 -1],  G = [1 0 0; .5 .5 .5; .5 -.5 .5; 0 0 1],
//   A^T = [1 1 1 0; 0 1 -1 -1]
// the cross-correlation of d with a 3x3 kernel g is A^T [(G g G^T) .* (B^T d B)] A. Summing over
// input channels and the three time taps, component xi = (a, b) of the 16 is
//   M_xi[o, t] = sum_c sum_i V_xi[o, c, i] U_xi[c, t - 2 + i],
// U = B^T d B the transformed input, V = G g G^T the transformed weight: a causal (3,1,1)
// convolution of the component plane U_xi, run on the matrix cores by the linear conv kernel.
// This file holds the three memory-bound steps around those products: the weight transform
// (at pack time), the input transform and the output transform.
#include "common.h"

namespace wvd {

namespace {

__device__ __forceinline__ float wload(const void* w, int bf, int64_t i) {
  return bf ? bf16_to_f32(((const bf16_t*)w)[i]) : ((const float*)w)[i];
}

// Raw weight [Co][Ci][3][3][3] -> 16 component weights in the linear kernel's packed layout,
// [16][Npad][3 time taps][Cip] bf16: V_xi[n][i][c] = (G g G^T)[a][b] with g = W[n][c][i][.][.],
// in fp32, rounded once.
__global__ void wino_pack_kernel(const void* __restrict__ w, int w_bf16, int Co, int Ci, int Npad, int Cip,
                                 bf16_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = (int64_t)Npad * 3 * Cip;
  if (idx >= 16 * per) return;
  const int xi = (int)(idx / per);
  const int64_t rem = idx - xi * per;
  const int c = (int)(rem % Cip);
  const int i = (int)((rem / Cip) % 3);
  const int n = (int)(rem / ((int64_t)Cip * 3));
  const int a = xi >> 2, b = xi & 3;
  float v = 0.0f;
  if (n < Co && c < Ci) {
    const float G[4][3] = {{1.0f, 0.0f, 0.0f}, {0.5f, 0.5f, 0.5f}, {0.5f, -0.5f, 0.5f}, {0.0f, 0.0f, 1.0f}};
    const int64_t base = (((int64_t)n * Ci + c) * 3 + i) * 9;
    for (int r = 0; r < 3; ++r) {
      float row = 0.0f;  // (g G^T)[r][b]
      for (int s = 0; s < 3; ++s) row += wload(w, w_bf16, base + r * 3 + s) * G[b][s];
      v += G[a][r] * row;
    }
  }
  out[idx] = (bf16_t)f32_to_bf16(v);
}

// One thread: frame f of the Th + T input frames (the history first), tile (ty, tx), 4 channels
// from c. Reads the 4x4 tile (8 bytes per position), writes its 16 components (8 bytes each) to
// U [16][Th + T][tH][tW][C]: consecutive threads take consecutive channel groups, so a wave's
// loads and stores are contiguous runs.
__global__ __launch_bounds__(256) void wino_in_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ hist,
                                                      int T, int Th, int H, int W, int C, int tH, int tW,
                                                      bf16_t* __restrict__ U) {
  const int cg = C >> 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int Tt = Th + T;
  const int64_t total = (int64_t)Tt * tH * tW * cg;
  if (idx >= total) return;
  const int c4 = (int)(idx % cg);
  int64_t r = idx / cg;
  const int tx = (int)(r % tW);
  r /= tW;
  const int ty = (int)(r % tH);
  const int f = (int)(r / tH);
  const int64_t fe = (int64_t)H * W * C;
  const bf16_t* src = f < Th ? hist + (int64_t)f * fe : x + (int64_t)(f - Th) * fe;
  float d[4][4][4];  // [row][col][channel]
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int h = 2 * ty - 1 + rr;
#pragma unroll
    for (int ss = 0; ss < 4; ++ss) {
      const int w = 2 * tx - 1 + ss;
      uint2 v = make_uint2(0u, 0u);
      if (h >= 0 && h < H && w >= 0 && w < W) v = *(const uint2*)(src + ((int64_t)h * W + w) * C + c4 * 4);
      d[rr][ss][0] = bf16_lo(v.x);
      d[rr][ss][1] = bf16_hi(v.x);
      d[rr][ss][2] = bf16_lo(v.y);
      d[rr][ss][3] = bf16_hi(v.y);
    }
  }
  const int64_t plane = (int64_t)Tt * tH * tW * C;
  bf16_t* dst = U + (((int64_t)f * tH + ty) * tW + tx) * C + c4 * 4;
  // e = B^T d (rows), then U = e B (columns)
  float e[4][4][4];
#pragma unroll
  for (int ss = 0; ss < 4; ++ss)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      e[0][ss][k] = d[0][ss][k] - d[2][ss][k];
      e[1][ss][k] = d[1][ss][k] + d[2][ss][k];
      e[2][ss][k] = d[2][ss][k] - d[1][ss][k];
      e[3][ss][k] = d[1][ss][k] - d[3][ss][k];
    }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    float u[4][4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      u[0][k] = e[a][0][k] - e[a][2][k];
      u[1][k] = e[a][1][k] + e[a][2][k];
      u[2][k] = e[a][2][k] - e[a][1][k];
      u[3][k] = e[a][1][k] - e[a][3][k];
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      uint2 o;
      o.x = pack_bf16x2(u[b][0], u[b][1]);
      o.y = pack_bf16x2(u[b][2], u[b][3]);
      *(uint2*)(dst + (int64_t)(a * 4 + b) * plane) = o;
    }
  }
}

// One thread: frame t, tile (ty, tx), 4 channels from c. Reads the 16 component products
// M [16][T][tH][tW][Co] (fp32), forms A^T M A (2x2 outputs) + bias (+ residual), rounds once and
// writes the outputs that lie inside the frame.
__global__ __launch_bounds__(256) void wino_out_kernel(const float* __restrict__ M, int T, int tH, int tW, int Co,
                                                       const float* __restrict__ bias, const bf16_t* __restrict__ res,
                                                       bf16_t* __restrict__ y, int H, int W) {
  const int cg = Co >> 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)T * tH * tW * cg;
  if (idx >= total) return;
  const int c4 = (int)(idx % cg);
  int64_t r = idx / cg;
  const int tx = (int)(r % tW);
  r /= tW;
  const int ty = (int)(r % tH);
  const int t = (int)(r / tH);
  const int64_t plane = (int64_t)T * tH * tW * Co;
  const float* src = M + (((int64_t)t * tH + ty) * tW + tx) * Co + c4 * 4;
  float m[4][4][4];
#pragma unroll
  for (int xi = 0; xi < 16; ++xi) {
    const float4 v = *(const float4*)(src + xi * plane);
    m[xi >> 2][xi & 3][0] = v.x;
    m[xi >> 2][xi & 3][1] = v.y;
    m[xi >> 2][xi & 3][2] = v.z;
    m[xi >> 2][xi & 3][3] = v.w;
  }
  float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (bias) {
    const float4 b4 = *(const float4*)(bias + c4 * 4);
    bv[0] = b4.x;
    bv[1] = b4.y;
    bv[2] = b4.z;
    bv[3] = b4.w;
  }
  // q = A^T m (rows), then Y = q A (columns)
  float q[2][4][4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      q[0][b][k] = m[0][b][k] + m[1][b][k] + m[2][b][k];
      q[1][b][k] = m[1][b][k] - m[2][b][k] - m[3][b][k];
    }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int h = 2 * ty + p;
    if (h >= H) continue;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int w = 2 * tx + qq;
      if (w >= W) continue;
      float v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        v[k] = (qq == 0 ? q[p][0][k] + q[p][1][k] + q[p][2][k] : q[p][1][k] - q[p][2][k] - q[p][3][k]) + bv[k];
      const int64_t o = (((int64_t)t * H + h) * W + w) * Co + c4 * 4;
      if (res) {
        const uint2 rv = *(const uint2*)(res + o);
        v[0] += bf16_lo(rv.x);
        v[1] += bf16_hi(rv.x);
        v[2] += bf16_lo(rv.y);
        v[3] += bf16_hi(rv.y);
      }
      uint2 out;
      out.x = pack_bf16x2(v[0], v[1]);
      out.y = pack_bf16x2(v[2], v[3]);
      *(uint2*)(y + o) = out;
    }
  }
}

unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_wino_pack(const void* w, int w_bf16, int Co, int Ci, int Npad, int Cip, bf16_t* out, hipStream_t s) {
  const int64_t n = (int64_t)16 * Npad * 3 * Cip;
  hipLaunchKernelGGL(wino_pack_kernel, dim3(blocks_for(n)), dim3(256), 0, s, w, w_bf16, Co, Ci, Npad, Cip, out);
  return hipGetLastError();
}

hipError_t launch_wino_in(const bf16_t* x, const bf16_t* hist, int T, int Th, int H, int W, int C, bf16_t* U,
                          hipStream_t s) {
  const int tH = (H + 1) / 2, tW = (W + 1) / 2;
  const int64_t n = (int64_t)(T + Th) * tH * tW * (C / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(wino_in_kernel, dim3(blocks_for(n)), dim3(256), 0, s, x, hist, T, Th, H, W, C, tH, tW, U);
  return hipGetLastError();
}

hipError_t launch_wino_out(const float* M, int T, int H, int W, int Co, const float* bias, const bf16_t* res,
                           bf16_t* y, hipStream_t s) {
  const int tH = (H + 1) / 2, tW = (W + 1) / 2;
  const int64_t n = (int64_t)T * tH * tW * (Co / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(wino_out_kernel, dim3(blocks_for(n)), dim3(256), 0, s, M, T, tH, tW, Co, bias, res, y, H, W);
  return hipGetLastError();
}

}  // namespace wvd
