// Implicit-GEMM causal convolution on the gfx950 matrix cores (bf16 operands, fp32 accumulation).
//
// The convolution (the causal conv part of the FastVideo compare page "[perf] PAN2 sampling:
// Wan2.2 VAE decode kernel, split decode, fused DiT kernels") is computed as a GEMM
//   D[n][m] = sum_k Wpk[n][k] * A[k][m]
// where m runs over the output positions (t, h, w) of the input grid, n over the output
// channels, and k over (tap, input channel). No im2col tensor exists: every lane reads its
// operand straight from the NTHWC activation, shifted by the tap's (dt, dh, dw) offset. A tap that
// lands before frame 0 reads the history tensor (the frames of the previous chunk); one that
// lands outside the frame or before the history reads zero.
//
// Work split: a workgroup owns BN = 32*NB output channels and BM = WAVES*MB*32 positions; each
// wave owns all BN channels and its own MB*32 positions, so the activation operand is private
// to a wave and goes from memory straight into registers (16 contiguous bytes = 8 channels of
// one position per lane, which is exactly one operand slice of v_mfma_f32_32x32x16_bf16). The
// weight tile is shared by the waves and staged through LDS, double-buffered, one barrier per
// K step of 32 channels. With the weights as the MFMA's first operand, each lane ends up holding
// 4 consecutive output channels of one position, stored as one 8-byte write.
//
// Output mapping (time-interleaved upsampling, phase-interleaved x2 spatial upsampling, NCTHW
// video) is applied in the epilogue together with the bias and an optional residual add, and
// the result is rounded to bf16 once.
#include <algorithm>

#include "common.h"

namespace wvd {

namespace {

constexpr int LDS_ROW = 40;  // bf16 per LDS row: 32 channels + 8 pad (80 bytes: no bank conflicts)

struct LoadCursor {
  int tap, chunk;
};

template <int NB, int MB, int WAVES>
__global__ __launch_bounds__(WAVES * 64, 1) void conv_mfma_kernel(const ConvProblem p) {
  constexpr int BN = NB * 32;
  constexpr int BM = WAVES * MB * 32;
  constexpr int NT = WAVES * 64;
  constexpr int WPIECES = BN * 4;  // 16-byte pieces of one weight K step
  constexpr int WLOADS = (WPIECES + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2][BN * LDS_ROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int phase = blockIdx.z;

  const int HW = p.H * p.W;
  const int M = p.T * HW;
  const int numM = (M + BM - 1) / BM;
  const int numN = (p.Npad + BN - 1) / BN;
  const int total = numM * numN;

  // XCD-aware tile order: the hardware deals workgroups round-robin to the 8 XCDs; give each
  // XCD one contiguous range of tiles so neighbouring tiles (which share halo rows and the
  // same weights) meet in the same L2.
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int q8 = total >> 3, r8 = total & 7;
  const int lin = xcd * q8 + (xcd < r8 ? xcd : r8) + local;
  const int mt = lin / numN, nt = lin - (lin / numN) * numN;
  const int n0 = nt * BN;
  const int mbase = mt * BM + wave * (MB * 32);

  int pt[MB], ph[MB], pw[MB];
  bool pv[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = mbase + mb * 32 + l32;
    pv[mb] = m < M;
    const int mm = pv[mb] ? m : 0;
    const int t = mm / HW;
    const int r = mm - t * HW;
    const int h = r / p.W;
    pt[mb] = t;
    ph[mb] = h;
    pw[mb] = r - h * p.W;
  }

  const int nchunks = p.Cip >> 5;
  const int nk = p.ntaps * nchunks;
  const int64_t frame_elems = (int64_t)HW * p.Ci;
  const int64_t wrow = (int64_t)p.ntaps * p.Cip;
  const bf16_t* wbase = p.wpk + ((int64_t)phase * p.Npad + n0) * wrow;
  const int pa = (p.phases == 4) ? (phase >> 1) : 0;
  const int pb = (p.phases == 4) ? (phase & 1) : 0;

  // Per-tap row pointers of this lane (recomputed when the load cursor enters a new tap).
  const bf16_t* rowp[MB];
  auto set_tap = [&](int tap) {
    int dt, dh, dw;
    if (p.phases == 4) {
      dt = 0;
      dh = (tap >> 1) + pa - 1;
      dw = (tap & 1) + pb - 1;
    } else {
      const int khw = p.kh * p.kw;
      const int i = tap / khw;
      const int j = (tap - i * khw) / p.kw;
      dt = i - 2 * (p.kt >> 1);
      dh = j - (p.kh >> 1);
      dw = tap - i * khw - j * p.kw - (p.kw >> 1);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int s = pt[mb] + dt;
      const int hh = ph[mb] + dh;
      const int ww = pw[mb] + dw;
      const bool ok = pv[mb] && hh >= 0 && hh < p.H && ww >= 0 && ww < p.W && s >= -p.Th;
      const bf16_t* base = (s >= 0) ? p.x + (int64_t)s * frame_elems : p.hist + (int64_t)(s + p.Th) * frame_elems;
      rowp[mb] = ok ? base + (int64_t)(hh * p.W + ww) * p.Ci + half * 16 : nullptr;
    }
  };

  typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
  u32x4 areg[2][MB][2];
  u32x4 wreg[WLOADS];

  auto load_act = [&](u32x4 (&dst)[MB][2], int chunk) {
    const int c = chunk * 32 + half * 16;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (rowp[mb] && c + s * 8 < p.Ci) v = *(const u32x4*)(rowp[mb] + chunk * 32 + s * 8);
        dst[mb][s] = v;
      }
    }
  };
  auto load_w = [&](int tap, int chunk) {
#pragma unroll
    for (int i = 0; i < WLOADS; ++i) {
      const int q = tid + i * NT;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (q < WPIECES) {
        const int row = q >> 2, piece = q & 3;
        if (n0 + row < p.Npad) v = *(const u32x4*)(wbase + row * wrow + tap * p.Cip + chunk * 32 + piece * 8);
      }
      wreg[i] = v;
    }
  };
  auto store_w = [&](int buf) {
#pragma unroll
    for (int i = 0; i < WLOADS; ++i) {
      const int q = tid + i * NT;
      if (q < WPIECES) {
        const int row = q >> 2, piece = q & 3;
        *(u32x4*)(&lds[buf][row * LDS_ROW + piece * 8]) = wreg[i];
      }
    }
  };

  floatx16 acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.0f;

  auto compute = [&](const u32x4 (&a)[MB][2], int buf) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 wf[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x4 v = *(const u32x4*)(&lds[buf][(nb * 32 + l32) * LDS_ROW + half * 16 + s * 8]);
        wf[nb] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 af = __builtin_bit_cast(bf16x8, a[mb][s]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[nb], af, acc[nb][mb], 0, 0, 0);
      }
    }
  };

  // Prologue: K step 0.
  LoadCursor cur = {0, 0};
  set_tap(0);
  load_act(areg[0], 0);
  load_w(0, 0);
  store_w(0);
  __syncthreads();

  auto advance = [&](LoadCursor& c) {
    if (++c.chunk == nchunks) {
      c.chunk = 0;
      ++c.tap;
      set_tap(c.tap);
    }
  };

  // Main loop, unrolled by two so the register double buffer is indexed statically; an odd
  // last K step runs after the loop (no exit from the middle of the body, which would split
  // the accumulators' live ranges).
  int k = 0;
  for (; k + 2 <= nk; k += 2) {
    advance(cur);
    load_act(areg[1], cur.chunk);
    load_w(cur.tap, cur.chunk);
    compute(areg[0], 0);
    store_w(1);
    __syncthreads();
    const bool more = k + 2 < nk;
    if (more) {
      advance(cur);
      load_act(areg[0], cur.chunk);
      load_w(cur.tap, cur.chunk);
    }
    compute(areg[1], 1);
    if (more) store_w(0);
    __syncthreads();
  }
  if (k < nk) compute(areg[0], 0);

  // Epilogue: lane holds, per (nb, mb, g), channels n0 + nb*32 + g*8 + half*4 + {0..3} of
  // position mbase + mb*32 + l32. Scheduling barriers keep one (mb, nb) block in flight at a
  // time so the accumulators are not all copied out of the AGPRs at once.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const bool valid = pv[mb];
    const int orow = p.hmul * ph[mb] + pa;
    const int ocol = p.wmul * pw[mb] + pb;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + nb * 32 + g * 8 + half * 4;
        if (!valid || n >= p.N) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[nb][mb][g * 4 + e] + ((p.bias && n + e < p.N) ? p.bias[n + e] : 0.0f);
        if (!p.y_ncthw) {
          // the 4 channels share a frame and are contiguous (nsplit is a multiple of 4 here)
          const int f = p.fbase + p.fmul * pt[mb] + n / p.nsplit;
          const int nc = n % p.nsplit;
          const int64_t idx = (((int64_t)f * p.Ho + orow) * p.Wo + ocol) * p.nsplit + nc;
          if (p.res) {
            const uint2 r = *(const uint2*)(p.res + idx);
            v[0] += bf16_lo(r.x);
            v[1] += bf16_hi(r.x);
            v[2] += bf16_lo(r.y);
            v[3] += bf16_hi(r.y);
          }
          uint2 o;
          o.x = pack_bf16x2(v[0], v[1]);
          o.y = pack_bf16x2(v[2], v[3]);
          *(uint2*)(p.y + idx) = o;
        } else {
          const int f = p.fbase + pt[mb];
          const int64_t pix = ((int64_t)f * p.Ho + orow) * p.Wo + ocol;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < p.N) p.y[(int64_t)(n + e) * p.y_cstride + pix] = (bf16_t)f32_to_bf16(v[e]);
        }
      }
    }
  }
}

struct ConfigEntry {
  const char* name;
  int nb, mb, waves;
  void (*kernel)(const ConvProblem);
};

#define WVD_CONV_CONFIG(NB, MB, W) \
  { "conv_mfma_n" #NB "_m" #MB "_w" #W, NB, MB, W, conv_mfma_kernel<NB, MB, W> }

const ConfigEntry kConfigs[] = {
    WVD_CONV_CONFIG(6, 2, 4),  // 192 x 256 tiles
    WVD_CONV_CONFIG(3, 4, 4),  // 96 x 512
    WVD_CONV_CONFIG(3, 1, 4),  // 96 x 128: small grids
    WVD_CONV_CONFIG(1, 4, 4),  // 32 x 512: a few output channels
    WVD_CONV_CONFIG(6, 1, 4),  // 192 x 128
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

int64_t blocks_for(const ConfigEntry& c, int64_t M, int Npad) {
  const int64_t bm = (int64_t)c.waves * c.mb * 32, bn = (int64_t)c.nb * 32;
  return ((M + bm - 1) / bm) * ((Npad + bn - 1) / bn);
}

// Largest tile whose grid still gives every CU at least one workgroup per phase.
int choose_config(int64_t M, int Npad, int phases) {
  const int64_t cus = 256;
  if (Npad <= 32) return 3;
  if (Npad % 192 == 0) {
    if (blocks_for(kConfigs[0], M, Npad) * phases >= cus) return 0;
    if (blocks_for(kConfigs[4], M, Npad) * phases >= cus) return 4;
    return 2;
  }
  if (Npad % 96 == 0) {
    if (blocks_for(kConfigs[1], M, Npad) * phases >= cus) return 1;
    return 2;
  }
  return 2;
}

}  // namespace

const char* conv_config_name(int id) { return (id >= 0 && id < kNumConfigs) ? kConfigs[id].name : "?"; }
int conv_config_count() { return kNumConfigs; }

hipError_t launch_conv_mfma(const ConvProblem& p, hipStream_t s, int* config_id) {
  const int64_t M = (int64_t)p.T * p.H * p.W;
  if (M == 0) return hipSuccess;
  const int id = choose_config(M, p.Npad, p.phases);
  const ConfigEntry& c = kConfigs[id];
  const int64_t blocks = blocks_for(c, M, p.Npad);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (config_id) *config_id = id;
  hipLaunchKernelGGL(c.kernel, dim3((unsigned)blocks, 1, p.phases), dim3(c.waves * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace wvd
