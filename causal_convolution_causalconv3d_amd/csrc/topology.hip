// Kernels of the real Wan2.2 decoder's extra parts (the FastVideo compare page "[perf] PAN2
// sampling: Wan2.2 VAE decode kernel, split decode, fused DiT kernels", reference.py: its part
// list and the functions attention, dup_up and unpatchify): the attention's row softmax and value
// transpose (its two products run on the matrix-core conv kernel as 1x1 convs whose weights are
// the frame's keys and transposed values), the DupUp3D shortcut add, and the unpatchify + clamp
// write of the video. All memory-bound; bf16 in and out, fp32 arithmetic, one rounding.
#include "common.h"

namespace wvd {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// P[r][c] = exp(scale * (S[r][c] - m_r)) / sum_c exp(scale * (S[r][c] - m_r)), m_r the row's
// maximum: the softmax of one query's scores (fp32 in, fp32 statistics, bf16 out). One
// 256-thread workgroup per row; the row is read three times (it stays in L2).
__global__ __launch_bounds__(256) void softmax_rows_kernel(const float* __restrict__ S, int64_t ld_s, int cols,
                                                           float scale, bf16_t* __restrict__ P, int64_t ld_p) {
  __shared__ float red[8];
  const int64_t row = blockIdx.x;
  const float* s = S + row * ld_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float m = -INFINITY;
  for (int c = tid; c < cols; c += 256) m = fmaxf(m, s[c]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float k = scale * 1.4426950408889634f;  // exp(scale * d) = exp2(k * d)
  float sum = 0.0f;
  for (int c = tid; c < cols; c += 256) sum += exp2f(k * (s[c] - m));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
  if (lane == 0) red[4 + wave] = sum;
  __syncthreads();
  const float inv = 1.0f / ((red[4] + red[5]) + (red[6] + red[7]));
  bf16_t* p = P + row * ld_p;
  for (int c = tid; c < cols; c += 256) p[c] = (bf16_t)f32_to_bf16(exp2f(k * (s[c] - m)) * inv);
}

// vt[c][r] = v[r][c] for r < R and 0 for R <= r < ldo: v [R][C], vt [C][ldo] (64 x 64 tiles
// through LDS, both sides coalesced).
__global__ __launch_bounds__(256) void transpose_pad_kernel(const bf16_t* __restrict__ v, int R, int C,
                                                            bf16_t* __restrict__ vt, int ldo) {
  __shared__ bf16_t tile[64][66];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < C) ? v[(int64_t)r * C + c] : (bf16_t)0;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < C && r < ldo) vt[(int64_t)c * ldo + r] = tile[tx][i];
  }
}

// DupUp3D added in place: y [To][2H][2W][Co] += dup(x [T][H][W][Ci]) with
// dup[c, ft*t + a, 2y + i, 2x + j] = x[(4*ft*c + 4a + 2i + j) / r, t, y, x], r = Co*ft*4/Ci, and
// output frame f holding (t, a) with f + fo = ft*t + a (fo = ft - 1 on the pass holding latent
// frame 0, whose first ft - 1 copies are dropped). One thread per output position and 8
// channels; the sum in fp32, one rounding.
__global__ __launch_bounds__(256) void dup_add_kernel(bf16_t* __restrict__ y, const bf16_t* __restrict__ x, int To,
                                                      int H, int W, int Ci, int Co, int ft, int fo, int r) {
  const int cg = Co >> 3;
  const int64_t n = (int64_t)To * (2 * H) * (2 * W) * cg;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int g = (int)(i % cg);
  int64_t pos = i / cg;
  const int X = (int)(pos % (2 * W));
  pos /= 2 * W;
  const int Y = (int)(pos % (2 * H));
  const int f = (int)(pos / (2 * H));
  const int fp = f + fo, t = fp / ft, a = fp - (fp / ft) * ft;
  const int sub = 4 * a + 2 * (Y & 1) + (X & 1);
  const bf16_t* xs = x + (((int64_t)t * H + (Y >> 1)) * W + (X >> 1)) * Ci;
  bf16_t* yp = y + i * 8;
  const u32x4 v = *(const u32x4*)yp;
  u32x4 o;
  if (r == 4 * ft) {
    // each output channel c reads input channel c (nearest copies): 8 contiguous channels
    const u32x4 d = *(const u32x4*)(xs + g * 8);
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(bf16_lo(v[q]) + bf16_lo(d[q]), bf16_hi(v[q]) + bf16_hi(d[q]));
  } else if (ft == 1 && r == 2) {
    // channel c reads 2c + i (i the row parity): every other channel of 16 contiguous ones
    const u32x4 d0 = *(const u32x4*)(xs + g * 16), d1 = *(const u32x4*)(xs + g * 16 + 8);
    const bool odd = (Y & 1) != 0;
    const uint32_t w[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a = odd ? bf16_hi(w[2 * q]) : bf16_lo(w[2 * q]);
      const float b = odd ? bf16_hi(w[2 * q + 1]) : bf16_lo(w[2 * q + 1]);
      o[q] = pack_bf16x2(bf16_lo(v[q]) + a, bf16_hi(v[q]) + b);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c0 = g * 8 + 2 * q;
      const float lo = bf16_lo(v[q]) + bf16_to_f32(xs[(4 * ft * c0 + sub) / r]);
      const float hi = bf16_hi(v[q]) + bf16_to_f32(xs[(4 * ft * (c0 + 1) + sub) / r]);
      o[q] = pack_bf16x2(lo, hi);
    }
  }
  *(u32x4*)yp = o;
}

// video[k][fbase + f][p*y + i][p*x + j] = out[f][y][x][(k*p + j)*p + i], clamped to [-1, 1] when
// `clamp`: out [T][h][w][colours * p * p] bf16 (NTHWC), video [colours][frames][p*h][p*w] bf16.
// One thread per low-res position.
__global__ __launch_bounds__(256) void unpatchify_kernel(const bf16_t* __restrict__ out, int T, int h, int w,
                                                         int colours, int patch, int clamp, bf16_t* __restrict__ video,
                                                         int64_t frames, int fbase) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * h * w) return;
  const int x = (int)(i % w);
  const int yy = (int)((i / w) % h);
  const int f = (int)(i / ((int64_t)w * h));
  const bf16_t* src = out + i * colours * patch * patch;
  const int64_t H = (int64_t)h * patch, Wd = (int64_t)w * patch;
  for (int k = 0; k < colours; ++k)
    for (int ii = 0; ii < patch; ++ii)
      for (int jj = 0; jj < patch; ++jj) {
        float v = bf16_to_f32(src[(k * patch + jj) * patch + ii]);
        if (clamp) v = fminf(fmaxf(v, -1.0f), 1.0f);
        video[((int64_t)k * frames + fbase + f) * H * Wd + ((int64_t)yy * patch + ii) * Wd + (int64_t)x * patch + jj] =
            (bf16_t)f32_to_bf16(v);
      }
}

unsigned blocks_of(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_softmax_rows(const float* S, int64_t ld_s, int rows, int cols, float scale, bf16_t* P, int64_t ld_p,
                               hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if (rows < 0 || cols < 0 || ld_s < cols || ld_p < cols) return hipErrorInvalidValue;
  hipLaunchKernelGGL(softmax_rows_kernel, dim3((unsigned)rows), dim3(256), 0, s, S, ld_s, cols, scale, P, ld_p);
  return hipGetLastError();
}

hipError_t launch_transpose_pad(const bf16_t* v, int R, int C, bf16_t* vt, int ldo, hipStream_t s) {
  if (R == 0 || C == 0) return hipSuccess;
  if (R < 0 || C < 0 || ldo < R) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_pad_kernel, dim3((unsigned)((ldo + 63) / 64), (unsigned)((C + 63) / 64)), dim3(256), 0,
                     s, v, R, C, vt, ldo);
  return hipGetLastError();
}

hipError_t launch_dup_add(bf16_t* y, const bf16_t* x, int To, int T, int H, int W, int Ci, int Co, int ft, int fo,
                          hipStream_t s) {
  if (To == 0) return hipSuccess;
  if (Co % 8 != 0 || ft < 1 || fo < 0 || fo >= ft || (Co * ft * 4) % Ci != 0 || To + fo > ft * T)
    return hipErrorInvalidValue;
  const int r = Co * ft * 4 / Ci;
  const int64_t n = (int64_t)To * (2 * H) * (2 * W) * (Co / 8);
  hipLaunchKernelGGL(dup_add_kernel, dim3(blocks_of(n)), dim3(256), 0, s, y, x, To, H, W, Ci, Co, ft, fo, r);
  return hipGetLastError();
}

hipError_t launch_unpatchify(const bf16_t* out, int T, int h, int w, int colours, int patch, int clamp, bf16_t* video,
                             int64_t frames, int fbase, hipStream_t s) {
  const int64_t n = (int64_t)T * h * w;
  if (n == 0) return hipSuccess;
  if (colours < 1 || patch < 1 || fbase < 0 || fbase + T > frames) return hipErrorInvalidValue;
  hipLaunchKernelGGL(unpatchify_kernel, dim3(blocks_of(n)), dim3(256), 0, s, out, T, h, w, colours, patch, clamp, video,
                     frames, fbase);
  return hipGetLastError();
}

}  // namespace wvd
