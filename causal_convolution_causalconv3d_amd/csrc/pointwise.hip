// Memory-bound kernels of libwvd: channel RMS norm + SiLU, layout conversion, weight packing.
#include "common.h"

namespace wvd {

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// ---------------------------------------------------------------------------------------------
// Channel RMS norm + SiLU on NTHWC bf16 (the RMS norm part of the FastVideo compare page "[perf]
// PAN2 sampling: Wan2.2 VAE decode kernel, split decode, fused DiT kernels", in the form
// y = gamma * x / sqrt(mean_c x^2 + eps), then SiLU). A position's C channels are spread over G
// lanes (G = C/8 rounded up to a power of two), 8 channels (16 bytes) per lane, so one wave
// normalises 64/G positions per step with a single 16-byte load and store per lane; the
// sum of squares is reduced across the G lanes with xor shuffles. fp32 statistics, one rounding.
// ---------------------------------------------------------------------------------------------
// Channels past 512 (64 lanes x 8) take KPL chunks of 8 per lane, chunk sub + k * G.
template <int G, int KPL>
__global__ __launch_bounds__(256) void norm_silu_kernel(const bf16_t* __restrict__ x, const float* __restrict__ gamma,
                                                        float eps, int silu, bf16_t* __restrict__ y,
                                                        int64_t positions, int C) {
  constexpr int PPW = 64 / G;  // positions per wave step
  const int lane = threadIdx.x & 63;
  const int sub = lane % G;    // first 8-channel chunk of the position
  const int slot = lane / G;   // which position of the step
  const int cv = C >> 3;       // chunks per position
  bool active[KPL];
  float g[KPL][8];
#pragma unroll
  for (int k = 0; k < KPL; ++k) {
    active[k] = sub + k * G < cv;
#pragma unroll
    for (int e = 0; e < 8; ++e) g[k][e] = active[k] ? gamma[(sub + k * G) * 8 + e] : 0.0f;
  }
  const float inv_c = 1.0f / (float)C;
  const int64_t wave_id = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  // U position steps per iteration, their loads issued together (more bytes in flight per lane)
  constexpr int U = (KPL == 1) ? 2 : 1;
  for (int64_t p0 = wave_id * PPW; p0 < positions; p0 += U * nwaves * PPW) {
    u32x4 v[U][KPL];
    int64_t pos[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      pos[u] = p0 + u * nwaves * PPW + slot;
#pragma unroll
      for (int k = 0; k < KPL; ++k) {
        v[u][k] = u32x4{0u, 0u, 0u, 0u};
        if (active[k] && pos[u] < positions) v[u][k] = *(const u32x4*)(x + pos[u] * C + (sub + k * G) * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float f[KPL][8];
      float ss = 0.0f;
#pragma unroll
      for (int k = 0; k < KPL; ++k) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f[k][2 * q] = bf16_lo(v[u][k][q]);
          f[k][2 * q + 1] = bf16_hi(v[u][k][q]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(f[k][e], f[k][e], ss);
      }
#pragma unroll
      for (int m = G / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
      const float r = rsqrtf(ss * inv_c + eps);
#pragma unroll
      for (int k = 0; k < KPL; ++k) {
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float a = f[k][2 * q] * r * g[k][2 * q];
          float b = f[k][2 * q + 1] * r * g[k][2 * q + 1];
          if (silu) {
            a = silu_f32(a);
            b = silu_f32(b);
          }
          o[q] = pack_bf16x2(a, b);
        }
        if (active[k] && pos[u] < positions) *(u32x4*)(y + pos[u] * C + (sub + k * G) * 8) = o;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Layout / dtype conversion NCTHW <-> NTHWC, fp32 <-> bf16 (boundary marshalling; one thread per
// output element).
// ---------------------------------------------------------------------------------------------
__global__ void convert_kernel(const void* __restrict__ x, int x_bf16, int x_ncthw, void* __restrict__ y, int y_bf16,
                               int y_ncthw, int C, int64_t THW) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= THW * C) return;
  int64_t c, p;
  if (y_ncthw) {
    c = i / THW;
    p = i - c * THW;
  } else {
    p = i / C;
    c = i - p * C;
  }
  const int64_t j = x_ncthw ? c * THW + p : p * C + c;
  float v = x_bf16 ? bf16_to_f32(((const bf16_t*)x)[j]) : ((const float*)x)[j];
  if (y_bf16)
    ((bf16_t*)y)[i] = (bf16_t)f32_to_bf16(v);
  else
    ((float*)y)[i] = v;
}

__device__ __forceinline__ float load_w(const void* w, int bf, int64_t i) {
  return bf ? bf16_to_f32(((const bf16_t*)w)[i]) : ((const float*)w)[i];
}

// Raw [Co][Ci][taps] -> [Npad][taps][Cip] bf16, zero padded.
__global__ void pack_conv_kernel(const void* __restrict__ w, int w_bf16, int Co, int Ci, int taps, int Npad, int Cip,
                                 bf16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)Npad * taps * Cip;
  if (i >= total) return;
  const int c = (int)(i % Cip);
  const int tap = (int)((i / Cip) % taps);
  const int n = (int)(i / ((int64_t)Cip * taps));
  float v = 0.0f;
  if (n < Co && c < Ci) v = load_w(w, w_bf16, ((int64_t)n * Ci + c) * taps + tap);
  out[i] = (bf16_t)f32_to_bf16(v);
}

// Raw 3x3 [Co][Ci][3][3] -> four 2x2 phase kernels [4][Npad][4][Cip]. Output parity a (rows) reads
// the low-res rows y + a - 1 and y + a; the 3x3 row taps that land on them are {0} and {1,2}
// for a = 0, {0,1} and {2} for a = 1 (the same for columns with parity b). Each phase tap is the
// fp32 sum of its 3x3 taps (row-major order), rounded once to bf16.
__global__ void pack_phase2x_kernel(const void* __restrict__ w, int w_bf16, int Co, int Ci, int Npad, int Cip,
                                    bf16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)4 * Npad * 4 * Cip;
  if (i >= total) return;
  const int c = (int)(i % Cip);
  const int tap = (int)((i / Cip) % 4);
  const int n = (int)((i / ((int64_t)Cip * 4)) % Npad);
  const int phase = (int)(i / ((int64_t)Cip * 4 * Npad));
  const int a = phase >> 1, b = phase & 1, u = tap >> 1, v = tap & 1;
  // taps of 3 that fall on low-res offset index u (0: first, 1: second) for parity a
  const int r_lo = (a == 0) ? (u == 0 ? 0 : 1) : (u == 0 ? 0 : 2);
  const int r_hi = (a == 0) ? (u == 0 ? 0 : 2) : (u == 0 ? 1 : 2);
  const int s_lo = (b == 0) ? (v == 0 ? 0 : 1) : (v == 0 ? 0 : 2);
  const int s_hi = (b == 0) ? (v == 0 ? 0 : 2) : (v == 0 ? 1 : 2);
  float acc = 0.0f;
  if (n < Co && c < Ci) {
    const int64_t base = ((int64_t)n * Ci + c) * 9;
    for (int r = r_lo; r <= r_hi; ++r)
      for (int s = s_lo; s <= s_hi; ++s) acc += load_w(w, w_bf16, base + r * 3 + s);
  }
  out[i] = (bf16_t)f32_to_bf16(acc);
}

__global__ void copy_f32_kernel(const float* __restrict__ src, float* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

unsigned grid_for(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

}  // namespace

hipError_t launch_norm_silu(const bf16_t* x, const float* gamma, float eps, int silu, bf16_t* y, int64_t positions,
                            int C, hipStream_t s) {
  if (positions == 0) return hipSuccess;
  const int cv = C / 8;
  if (C % 8 != 0 || cv > 64 * 4) return hipErrorInvalidValue;
  int G = 1;
  while (G < cv && G < 64) G *= 2;
  const int kpl = (cv + G - 1) / G;  // chunks per lane: 1 up to 512 channels
  const int ppb = 4 * (64 / G) * (kpl == 1 ? 2 : 1);  // positions per block iteration (U steps)
  int64_t blocks = (positions + ppb - 1) / ppb;
  if (blocks > 8192) blocks = 8192;
#define WVD_NORM_CASE(GG, KK) \
  if (G == GG && kpl == KK) { \
    hipLaunchKernelGGL((norm_silu_kernel<GG, KK>), dim3((unsigned)blocks), dim3(256), 0, s, x, gamma, eps, silu, y, positions, C); \
    return hipGetLastError(); \
  }
  WVD_NORM_CASE(1, 1)
  WVD_NORM_CASE(2, 1)
  WVD_NORM_CASE(4, 1)
  WVD_NORM_CASE(8, 1)
  WVD_NORM_CASE(16, 1)
  WVD_NORM_CASE(32, 1)
  WVD_NORM_CASE(64, 1)
  WVD_NORM_CASE(64, 2)
  WVD_NORM_CASE(64, 3)
  WVD_NORM_CASE(64, 4)
#undef WVD_NORM_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_convert(const void* x, int x_bf16, int x_ncthw, void* y, int y_bf16, int y_ncthw, int C, int T, int H,
                          int W, hipStream_t s) {
  const int64_t THW = (int64_t)T * H * W;
  const int64_t n = THW * C;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(convert_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, x, x_bf16, x_ncthw, y, y_bf16, y_ncthw, C,
                     THW);
  return hipGetLastError();
}

hipError_t launch_pack_conv(const void* w, int w_bf16, int Co, int Ci, int ntaps_raw, int Npad, int Cip, bf16_t* out,
                            hipStream_t s) {
  const int64_t n = (int64_t)Npad * ntaps_raw * Cip;
  hipLaunchKernelGGL(pack_conv_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, w, w_bf16, Co, Ci, ntaps_raw, Npad,
                     Cip, out);
  return hipGetLastError();
}

hipError_t launch_pack_phase2x(const void* w, int w_bf16, int Co, int Ci, int Npad, int Cip, bf16_t* out,
                               hipStream_t s) {
  const int64_t n = (int64_t)16 * Npad * Cip;
  hipLaunchKernelGGL(pack_phase2x_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, w, w_bf16, Co, Ci, Npad, Cip, out);
  return hipGetLastError();
}

hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_f32_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

}  // namespace wvd
