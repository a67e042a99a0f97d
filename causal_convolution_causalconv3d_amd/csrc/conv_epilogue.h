// Epilogue of the matrix-core convolution kernels: bias, optional residual add or fused channel
// RMS norm (+ SiLU), the output mapping of ConvProblem, and one bf16 (or fp32) rounding.
#pragma once

#include "common.h"

namespace wvd {

// Four consecutive per-channel values v[n .. n+3] (n a multiple of 4) as one 16-byte load when the
// array is 16-byte aligned and all four exist, else element by element; entries >= N are 0.
__device__ __forceinline__ float4 load4(const float* v, int n, int N) {
  if (!v) return make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if ((((uintptr_t)v & 15u) == 0) & (n + 3 < N)) return *(const float4*)(v + n);
  float4 r;
  r.x = n + 0 < N ? v[n + 0] : 0.0f;
  r.y = n + 1 < N ? v[n + 1] : 0.0f;
  r.z = n + 2 < N ? v[n + 2] : 0.0f;
  r.w = n + 3 < N ? v[n + 3] : 0.0f;
  return r;
}

// A per-channel array pointer the compiler must treat as new at each call: the epilogue runs
// once per tile inside a tile loop, and loads of bias and gamma hoisted out of that loop would
// hold their registers through the whole reduction.
template <typename T>
__device__ __forceinline__ const T* opaque(const T* ptr) {
  asm volatile("" : "+s"(ptr));
  return ptr;
}

// NORM selects the fused RMS norm (+ SiLU) epilogue (p.norm_gamma set), instantiated separately so
// that its registers do not weigh on the plain kernels. The lane holds, per (nb, mb, g), channels n0 + nb*32 + g*8 + half*4 + {0..3} of position
// (ph[mb], pw[mb]) of frame tf (valid when pv[mb]); (pa, pb) is the output phase. Scheduling
// barriers keep one (mb, nb) block in flight at a time so the accumulators are not all copied
// out of the AGPRs at once.
template <int NB, int MB, bool NORM>
__device__ __forceinline__ void conv_epilogue(const ConvProblem& p, floatx16 (&acc)[NB][MB], const int (&ph)[MB],
                                              const int (&pw)[MB], const bool (&pv)[MB], int tf, int n0, int pa,
                                              int pb, int half) {
  const float* bias = opaque(p.bias);
  const float* gamma = opaque(p.norm_gamma);
  asm volatile("" : "+v"(half));
  if constexpr (NORM) {
    // Fused channel RMS norm (+ SiLU) of the conv output: the workgroup holds every channel of
    // its positions (one N tile), split between lanes l and l ^ 32, so the per-position sum of
    // squares is this lane's part plus one cross-lane exchange. fp32 statistics on the unrounded
    // sums, one bf16 rounding of the activated value.
    // (launched only with N % 8 == 0 and 16-byte aligned bias and gamma, so an 8-channel group c
    // .. c+7 is wholly in or out of range: wave-uniform tests; channels in [N, Npad) have zero
    // weights and bias, so their accumulators are 0)
    const float inv_n = 1.0f / (float)p.N;
    float ssm[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) ssm[mb] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = nb * 32 + g * 8;
        if (c >= p.N) continue;
        const float4 b4 = bias ? *(const float4*)(bias + c + half * 4) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = acc[nb][mb][g * 4 + e] + bv[e];
            acc[nb][mb][g * 4 + e] = v;
            ssm[mb] = fmaf(v, v, ssm[mb]);
          }
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float ss = ssm[mb];
      ss += __shfl_xor(ss, 32, 64);
      const float r = rsqrtf(ss * inv_n + p.norm_eps);
      const bool valid = pv[mb];
      const int orow = p.hmul * ph[mb] + pa;
      const int ocol = p.wmul * pw[mb] + pb;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = nb * 32 + g * 8 + half * 4;
          if ((nb * 32 + g * 8 >= p.N) || !valid) continue;
          const float4 gm = *(const float4*)(gamma + n);
          const float gv[4] = {gm.x, gm.y, gm.z, gm.w};
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = acc[nb][mb][g * 4 + e] * r * gv[e];
            if (p.norm_silu) v[e] = silu_f32(v[e]);
          }
          const int f = p.fbase + p.fmul * tf + p.fstride * (n / p.nsplit);
          const int nc = n % p.nsplit;
          const int64_t idx = (((int64_t)f * p.Ho + orow) * p.Wo + ocol) * p.nsplit + nc;
          uint2 o;
          o.x = pack_bf16x2(v[0], v[1]);
          o.y = pack_bf16x2(v[2], v[3]);
          *(uint2*)((bf16_t*)p.y + idx) = o;
        }
      }
    }
    return;
  }
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
        const float4 b4 = load4(bias, n, p.N);
        const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[nb][mb][g * 4 + e] + bv[e];
        // the 4 channels share a frame and are contiguous (nsplit is a multiple of 4)
        const int f = p.fbase + p.fmul * tf + p.fstride * (n / p.nsplit);
        const int nc = n % p.nsplit;
        const int64_t idx = (((int64_t)f * p.Ho + orow) * p.Wo + ocol) * p.nsplit + nc;
        if (p.y_f32) {
          float4 o;
          o.x = n + 0 < p.N ? v[0] : 0.0f;
          o.y = n + 1 < p.N ? v[1] : 0.0f;
          o.z = n + 2 < p.N ? v[2] : 0.0f;
          o.w = n + 3 < p.N ? v[3] : 0.0f;
          *(float4*)((float*)p.y + idx) = o;
        } else {
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
          *(uint2*)((bf16_t*)p.y + idx) = o;
        }
      }
    }
  }
}

// Output index of channel n (a multiple of 4) at output row orow, column ocol of frame tf.
__device__ __forceinline__ int64_t out_index(const ConvProblem& p, int tf, int n, int orow, int ocol) {
  const int fs = p.fstride ? n / p.nsplit : 0;
  const int f = p.fbase + p.fmul * tf + p.fstride * fs;
  const int nc = n - fs * p.nsplit;
  return (((int64_t)f * p.Ho + orow) * p.Wo + ocol) * p.nsplit + nc;
}

// Epilogue through LDS (p.staged: bf16 output, N and nsplit multiples of 8, y and res 16-byte
// aligned). The accumulator layout scatters a store instruction over 32 positions (8 bytes per
// lane, one position's channels 2 * nsplit bytes apart), so instead each wave writes its values
// into a private LDS area, one row of 32 positions and up to 96 channels at a time, and then
// stores 16 contiguous bytes per lane, consecutive lanes on consecutive addresses. The residual
// comes in the same coalesced way and is added in fp32 before the single rounding. `stage` holds
// 32 * PS bytes for this wave alone (PS = 16-byte padded position stride); the same values and
// rounding as conv_epilogue. A pass covers NBP 32-channel blocks (NBP divides NB).
template <int NBP_>
struct StagedShape {
  static constexpr int NBP = NBP_;              // 32-channel blocks per pass
  static constexpr int CHP = NBP * 4;           // 16-byte chunks of a position in one pass
  static constexpr int PS = NBP * 64 + 16;      // LDS bytes per position
  static constexpr int CPL = 32 * CHP / 64;     // chunks per lane and pass
  static constexpr int BYTES = 32 * PS;         // one wave's LDS area
  static_assert((32 * CHP) % 64 == 0, "pass shape");
};

// A 16-byte store marked non-temporal: the conv outputs are streamed out (a layer's output is
// read back by the next kernel, long after the L2 has turned over), so they should not displace
// the input patches and weights the other tiles are still reading from L2. (Measured on the
// decode: 1-2 % faster overall, 8 % on the 192-channel x2 phase conv with its two outputs.)
__device__ __forceinline__ void store_stream16(bf16_t* dst, uint4 v) {
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4v, v), (u32x4v*)dst);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// DUAL (with NORM): the residual (p.res, optional) is added before the norm's statistics, and the
// pre-norm value (bias and residual added) is stored to p.y_pre beside the activated value in p.y:
// a residual block's output and the next block's SiLU(norm1(.)) input from one epilogue.
// SC (with DUAL, 192 channels in one tile): instead of the pre-norm value, its 1x1 product with
// p.sc_w (96 outputs) plus p.sc_b goes to p.y_sc (see ConvProblem::y_sc); sc_lds holds p.sc_w's
// rows 196 elements apart.
template <int NB, int MB, bool NORM, int NBP, bool DUAL = false, bool SC = false>
__device__ __forceinline__ void conv_epilogue_staged(const ConvProblem& p, floatx16 (&acc)[NB][MB], const int (&ph)[MB],
                                                     int w0, int tf, int n0, int pa, int pb, int lane, char* stage,
                                                     const bf16_t* sc_lds = nullptr) {
  static_assert(!DUAL || NORM, "the dual store belongs to the fused norm");
  static_assert(!SC || (DUAL && NB == 6 && NBP == 3), "the shortcut product: 192 channels in, 96-channel passes");
  const float* bias = opaque(p.bias);
  const float* gamma = opaque(p.norm_gamma);
  asm volatile("" : "+v"(lane));  // (the chunk indices below are per call, not hoisted)
  using S = StagedShape<NBP>;
  static_assert(NB % NBP == 0, "pass shape");
  constexpr int NPG = NB / S::NBP;  // passes per row
  const int half = lane >> 5, l32 = lane & 31;
  float rs[MB];  // the norm's 1 / rms per row
  if constexpr (NORM) {
    // bias, then the per-position sum of squares over all channels (see conv_epilogue)
    const float inv_n = 1.0f / (float)p.N;
    float ssm[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) ssm[mb] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = nb * 32 + g * 8;
        if (c >= p.N) continue;
        const float4 b4 = bias ? *(const float4*)(bias + c + half * 4) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = acc[nb][mb][g * 4 + e] + bv[e];
            acc[nb][mb][g * 4 + e] = v;
            if constexpr (!DUAL) ssm[mb] = fmaf(v, v, ssm[mb]);
          }
      }
    }
    if constexpr (DUAL) {
      // + residual, read per row and pass the coalesced way through this wave's staging area
      // (the plain epilogue's order: (acc + bias) + residual), then the sum of squares
      if (p.res) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          if (ph[mb] >= p.H) continue;  // wave-uniform
          const int orow = p.hmul * ph[mb] + pa;
#pragma unroll
          for (int pg = 0; pg < NPG; ++pg) {
            const int cb = pg * S::NBP * 32;
            if (cb >= p.N) continue;
            __builtin_amdgcn_sched_barrier(0);
            uint4 r[S::CPL];
#pragma unroll
            for (int i = 0; i < S::CPL; ++i) {
              const int j = i * 64 + lane, q = j / S::CHP, c = j - (j / S::CHP) * S::CHP;
              const int n = cb + c * 8, w = w0 + q;
              r[i] = (w < p.W && n < p.N) ? *(const uint4*)(p.res + out_index(p, tf, n, orow, p.wmul * w + pb))
                                          : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int i = 0; i < S::CPL; ++i) {
              const int j = i * 64 + lane, q = j / S::CHP, c = j - (j / S::CHP) * S::CHP;
              *(uint4*)(stage + q * S::PS + c * 16) = r[i];
            }
            wave_lds_sync();
#pragma unroll
            for (int nl = 0; nl < S::NBP; ++nl) {
              const int nb = pg * S::NBP + nl;
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                if (nb * 32 + g * 8 >= p.N) continue;
                const uint2 rr = *(const uint2*)(stage + l32 * S::PS + (nl * 32 + g * 8 + half * 4) * 2);
                acc[nb][mb][g * 4 + 0] += bf16_lo(rr.x);
                acc[nb][mb][g * 4 + 1] += bf16_hi(rr.x);
                acc[nb][mb][g * 4 + 2] += bf16_lo(rr.y);
                acc[nb][mb][g * 4 + 3] += bf16_hi(rr.y);
              }
            }
            wave_lds_sync();
          }
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) ssm[mb] = fmaf(acc[nb][mb][r], acc[nb][mb][r], ssm[mb]);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const float ss = ssm[mb] + __shfl_xor(ssm[mb], 32, 64);
      rs[mb] = rsqrtf(ss * inv_n + p.norm_eps);
    }
  }
  if constexpr (SC) {
    // The shortcut's 96 x 192 product on the matrix cores, per row of 32 positions: the
    // accumulators, rounded to bf16 as the pre-norm store would round them, are the second
    // operand as they lie (K16 step (nb, q): this lane's registers 8q .. 8q + 7 of block nb, i.e.
    // channels nb * 32 + (2q + j / 4) * 8 + half * 4 + j % 4 for j = 0 .. 7), and the first
    // operand reads each weight row (in LDS) in that channel order (two 8-byte pieces). Then
    // + bias, one rounding, and 16-byte stores through the staging area (one 96-channel pass).
    typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
    const float* bsc = opaque(p.sc_b);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (ph[mb] >= p.H) continue;  // wave-uniform
      const int orow = p.hmul * ph[mb] + pa;
      floatx16 sa[3];
#pragma unroll
      for (int ob = 0; ob < 3; ++ob)
#pragma unroll
        for (int r = 0; r < 16; ++r) sa[ob][r] = 0.0f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          __builtin_amdgcn_sched_barrier(0);
          u32x4 b;
#pragma unroll
          for (int i = 0; i < 4; ++i) b[i] = pack_bf16x2(acc[nb][mb][q * 8 + 2 * i], acc[nb][mb][q * 8 + 2 * i + 1]);
          u32x4 a[3];
#pragma unroll
          for (int ob = 0; ob < 3; ++ob) {
            const bf16_t* wr = sc_lds + (ob * 32 + l32) * 196 + nb * 32 + q * 16 + half * 4;
            const uint2 lo = *(const uint2*)wr, hi = *(const uint2*)(wr + 8);
            a[ob][0] = lo.x;
            a[ob][1] = lo.y;
            a[ob][2] = hi.x;
            a[ob][3] = hi.y;
          }
#pragma unroll
          for (int ob = 0; ob < 3; ++ob)
            sa[ob] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[ob]),
                                                             __builtin_bit_cast(bf16x8, b), sa[ob], 0, 0, 0);
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ob = 0; ob < 3; ++ob)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = ob * 32 + g * 8 + half * 4;
          const float4 b4 = bsc ? *(const float4*)(bsc + n) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          uint2 o;
          o.x = pack_bf16x2(sa[ob][g * 4 + 0] + b4.x, sa[ob][g * 4 + 1] + b4.y);
          o.y = pack_bf16x2(sa[ob][g * 4 + 2] + b4.z, sa[ob][g * 4 + 3] + b4.w);
          *(uint2*)(stage + l32 * S::PS + n * 2) = o;
        }
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < S::CPL; ++i) {
        const int j = i * 64 + lane, q = j / S::CHP, c = j - (j / S::CHP) * S::CHP;
        const int w = w0 + q;
        const uint4 o = *(const uint4*)(stage + q * S::PS + c * 16);
        const int64_t at = (((int64_t)(p.fbase + p.fmul * tf) * p.Ho + orow) * p.Wo + p.wmul * w + pb) * p.sc_co + c * 8;
        if (w < p.W) store_stream16(p.y_sc + at, o);
      }
      wave_lds_sync();
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (ph[mb] >= p.H) continue;  // the whole row is outside the frame (wave-uniform)
    const int orow = p.hmul * ph[mb] + pa;
#pragma unroll
    for (int pg = 0; pg < NPG; ++pg) {
      const int cb = n0 + pg * S::NBP * 32;
      if (cb >= p.N) continue;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (DUAL && !SC) {
        // the pre-norm value (bias and residual already in the accumulators), one rounding
#pragma unroll
        for (int nl = 0; nl < S::NBP; ++nl) {
          const int nb = pg * S::NBP + nl;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            if (nb * 32 + g * 8 >= p.N) continue;
            uint2 o;
            o.x = pack_bf16x2(acc[nb][mb][g * 4 + 0], acc[nb][mb][g * 4 + 1]);
            o.y = pack_bf16x2(acc[nb][mb][g * 4 + 2], acc[nb][mb][g * 4 + 3]);
            *(uint2*)(stage + l32 * S::PS + (nl * 32 + g * 8 + half * 4) * 2) = o;
          }
        }
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < S::CPL; ++i) {
          const int j = i * 64 + lane, q = j / S::CHP, c = j - (j / S::CHP) * S::CHP;
          const int n = cb + c * 8, w = w0 + q;
          const uint4 o = *(const uint4*)(stage + q * S::PS + c * 16);
          if (w < p.W && n < p.N) store_stream16(p.y_pre + out_index(p, tf, n, orow, p.wmul * w + pb), o);
        }
        wave_lds_sync();
      }
      if (!NORM && p.res) {
        uint4 r[S::CPL];
#pragma unroll
        for (int i = 0; i < S::CPL; ++i) {
          const int j = i * 64 + lane, q = j / S::CHP, c = j - (j / S::CHP) * S::CHP;
          const int n = cb + c * 8, w = w0 + q;
          r[i] = (w < p.W && n < p.N) ? *(const uint4*)(p.res + out_index(p, tf, n, orow, p.wmul * w + pb))
                                      : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int i = 0; i < S::CPL; ++i) {
          const int j = i * 64 + lane, q = j / S::CHP, c = j - (j / S::CHP) * S::CHP;
          *(uint4*)(stage + q * S::PS + c * 16) = r[i];
        }
        wave_lds_sync();
      }
#pragma unroll
      for (int nl = 0; nl < S::NBP; ++nl) {
        const int nb = pg * S::NBP + nl;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + nb * 32 + g * 8 + half * 4;
          if (n0 + nb * 32 + g * 8 >= p.N) continue;  // N % 8 == 0: wave-uniform
          float v[4];
          if constexpr (NORM) {
            const float4 gm = *(const float4*)(gamma + n);
            const float gv[4] = {gm.x, gm.y, gm.z, gm.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[e] = acc[nb][mb][g * 4 + e] * rs[mb] * gv[e];
              if (p.norm_silu) v[e] = silu_f32(v[e]);
            }
          } else {
            const float4 b4 = load4(bias, n, p.N);
            const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[nb][mb][g * 4 + e] + bv[e];
          }
          uint2* a = (uint2*)(stage + l32 * S::PS + (nl * 32 + g * 8 + half * 4) * 2);
          if (!NORM && p.res) {
            const uint2 r = *a;
            v[0] += bf16_lo(r.x);
            v[1] += bf16_hi(r.x);
            v[2] += bf16_lo(r.y);
            v[3] += bf16_hi(r.y);
          }
          uint2 o;
          o.x = pack_bf16x2(v[0], v[1]);
          o.y = pack_bf16x2(v[2], v[3]);
          *a = o;
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < S::CPL; ++i) {
        const int j = i * 64 + lane, q = j / S::CHP, c = j - (j / S::CHP) * S::CHP;
        const int n = cb + c * 8, w = w0 + q;
        const uint4 o = *(const uint4*)(stage + q * S::PS + c * 16);
        if (w < p.W && n < p.N) store_stream16((bf16_t*)p.y + out_index(p, tf, n, orow, p.wmul * w + pb), o);
      }
      wave_lds_sync();
    }
  }
}

}  // namespace wvd
