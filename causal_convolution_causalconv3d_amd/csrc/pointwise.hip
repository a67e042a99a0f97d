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
// A residual block's norm1 + SiLU and its 1x1 shortcut from one read of the block's input (the
// residual block of the FastVideo compare page's reference decoder: the input feeds both the
// normalised branch and, when the channel count changes, the 1x1 shortcut), for 384 input
// channels and up to 192 shortcut outputs. The separate passes read the input twice; here a
// workgroup keeps the shortcut weight in LDS and walks tiles of 256 positions, each wave 32 of
// them, and each lane loads the 192 channels of its position that the shortcut's matrix operand
// gives it (K step c, half h, register q: channels 32c + 16h + 8q .. + 7). From those registers
// it forms
//   * the norm: the 8-channel sums of squares added in the standalone norm's lane-reduction
//     order (chunks j and j ^ m for m = 32, 16, 8, 4 within the lane, 2 across the lane pair,
//     1 within the lane), so act equals that kernel's output bit for bit;
//   * the shortcut: W x on the matrix cores with the linear conv kernel's K order per
//     accumulator (K steps in order, register 0 then 1), + bias, one rounding, so sc equals
//     that kernel's output bit for bit.
// ---------------------------------------------------------------------------------------------
constexpr int NSC_C = 384;              // input channels
constexpr int NSC_KS = NSC_C / 32;      // 32-channel K steps
constexpr int NSC_WROW = NSC_C + 8;     // bf16 per LDS weight row (784 bytes: 16-byte reads of 16 rows on distinct banks)
constexpr int NSC_MAXN = 192;
constexpr int NSC_TILE = 256;           // positions per workgroup tile (8 waves x 32)

__global__ __launch_bounds__(512, 1) void norm_shortcut_kernel(const bf16_t* __restrict__ x, int64_t positions,
                                                               const float* __restrict__ gamma, float eps,
                                                               bf16_t* __restrict__ act, const bf16_t* __restrict__ wpk,
                                                               int N, const float* __restrict__ bias,
                                                               bf16_t* __restrict__ sc) {
  __shared__ __attribute__((aligned(16))) bf16_t wl[NSC_MAXN * NSC_WROW];
  __shared__ __attribute__((aligned(16))) float gl[NSC_C];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, l32 = lane & 31;
  // the packed 1x1 weight (rows of 384 channels) into LDS; gamma beside it
  for (int q = tid; q < N * (NSC_C / 8); q += 512) {
    const int n = q / (NSC_C / 8), k8 = q - n * (NSC_C / 8);
    *(u32x4*)(&wl[n * NSC_WROW + k8 * 8]) = *(const u32x4*)(wpk + (int64_t)n * NSC_C + k8 * 8);
  }
  for (int c = tid; c < NSC_C; c += 512) gl[c] = gamma[c];
  __syncthreads();
  const float inv_c = 1.0f / (float)NSC_C;
  const int64_t ntiles = (positions + NSC_TILE - 1) / NSC_TILE;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t pos = tile * NSC_TILE + wave * 32 + l32;
    const bool valid = pos < positions;
    const int64_t at = valid ? pos : 0;
    const bf16_t* xp = x + at * NSC_C + half * 16;
    u32x4 xr[NSC_KS][2];
#pragma unroll
    for (int c = 0; c < NSC_KS; ++c)
#pragma unroll
      for (int q = 0; q < 2; ++q) xr[c][q] = valid ? *(const u32x4*)(xp + c * 32 + q * 8) : u32x4{0u, 0u, 0u, 0u};
    // sum of squares of chunk j = 4c + 2 half + q (channels 8j .. 8j + 7, in order); chunks 48 ..
    // 63 of the standalone norm's 64 lanes hold nothing
    float sq[NSC_KS][2];
#pragma unroll
    for (int c = 0; c < NSC_KS; ++c)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = bf16_lo(xr[c][q][i]), b = bf16_hi(xr[c][q][i]);
          acc = fmaf(a, a, acc);
          acc = fmaf(b, b, acc);
        }
        sq[c][q] = acc;
      }
    // the reduction tree: j + 32 (chunk c + 8; none past chunk 47), j + 16 (c + 4), j + 8 (c + 2),
    // j + 4 (c + 1), then j ^ 2 (the other half of the lane pair) and j ^ 1 (q)
    float t[8][2], u[4][2], v[2][2], w[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int c = 0; c < 8; ++c) t[c][q] = sq[c][q] + (c + 8 < NSC_KS ? sq[c + 8][q] : 0.0f);
#pragma unroll
      for (int c = 0; c < 4; ++c) u[c][q] = t[c][q] + t[c + 4][q];
#pragma unroll
      for (int c = 0; c < 2; ++c) v[c][q] = u[c][q] + u[c + 2][q];
      w[q] = v[0][q] + v[1][q];
    }
    const float y0 = w[0] + __shfl_xor(w[0], 32, 64);
    const float y1 = w[1] + __shfl_xor(w[1], 32, 64);
    const float r = rsqrtf((y0 + y1) * inv_c + eps);
    // act = SiLU(gamma * x * r), one rounding (the standalone norm's arithmetic)
    bf16_t* ap = act + at * NSC_C + half * 16;
#pragma unroll
    for (int c = 0; c < NSC_KS; ++c)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        __builtin_amdgcn_sched_barrier(0);
        const int ch = c * 32 + half * 16 + q * 8;
        const float4 g0 = *(const float4*)(gl + ch), g1 = *(const float4*)(gl + ch + 4);
        const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // (unpacked again here: keeping the sums' fp32 copies of all 192 values would need as
          // many registers)
          uint32_t xv = xr[c][q][i];
          asm volatile("" : "+v"(xv));
          const float a = silu_f32(bf16_lo(xv) * r * g[2 * i]);
          const float b = silu_f32(bf16_hi(xv) * r * g[2 * i + 1]);
          o[i] = pack_bf16x2(a, b);
        }
        if (valid) *(u32x4*)(ap + c * 32 + q * 8) = o;
      }
    // sc = W x + bias in passes of up to 96 outputs (3 accumulator blocks); the lane ends with
    // outputs n0 + nb * 32 + g * 8 + half * 4 + {0..3} of its position
    bf16_t* sp = sc + at * N;
    for (int n0 = 0; n0 < N; n0 += 96) {
      const int nbs = (N - n0) / 32 < 3 ? (N - n0) / 32 : 3;  // (uniform)
      floatx16 acc[3];
#pragma unroll
      for (int nb = 0; nb < 3; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[nb][e] = 0.0f;
#pragma unroll
      for (int c = 0; c < NSC_KS; ++c) {
        // (one K step's weight fragments in flight at a time: the x registers fill half the budget)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int nb = 0; nb < 3; ++nb) {
            if (nb >= nbs) continue;
            const u32x4 a = *(const u32x4*)(&wl[(n0 + nb * 32 + l32) * NSC_WROW + c * 32 + half * 16 + q * 8]);
            acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                              __builtin_bit_cast(bf16x8, xr[c][q]), acc[nb], 0, 0, 0);
          }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < 3; ++nb) {
        if (nb >= nbs) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + nb * 32 + g * 8 + half * 4;
          const float4 b4 = bias ? *(const float4*)(bias + n) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          uint2 o;
          o.x = pack_bf16x2(acc[nb][g * 4 + 0] + b4.x, acc[nb][g * 4 + 1] + b4.y);
          o.y = pack_bf16x2(acc[nb][g * 4 + 2] + b4.z, acc[nb][g * 4 + 3] + b4.w);
          if (valid) *(uint2*)(sp + n) = o;
        }
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

bool norm_shortcut_supported(int C, int N) { return C == NSC_C && N % 32 == 0 && N >= 32 && N <= NSC_MAXN; }

hipError_t launch_norm_shortcut(const bf16_t* x, int64_t positions, int C, const float* gamma, float eps, bf16_t* act,
                                const bf16_t* wpk, int N, const float* bias, bf16_t* sc, hipStream_t s) {
  if (positions == 0) return hipSuccess;
  auto al16 = [](const void* q) { return ((uintptr_t)q & 15u) == 0; };
  if (!norm_shortcut_supported(C, N) || !x || !gamma || !act || !wpk || !sc || !al16(x) || !al16(gamma) || !al16(act) ||
      !al16(wpk) || !al16(sc) || !al16(bias) || positions > ((int64_t)1 << 40))
    return hipErrorInvalidValue;
  const int64_t tiles = (positions + NSC_TILE - 1) / NSC_TILE;
  const int64_t blocks = tiles < 256 ? tiles : 256;  // one workgroup per CU (the weight fills its LDS)
  hipLaunchKernelGGL(norm_shortcut_kernel, dim3((unsigned)blocks), dim3(512), 0, s, x, positions, gamma, eps, act, wpk,
                     N, bias, sc);
  return hipGetLastError();
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
