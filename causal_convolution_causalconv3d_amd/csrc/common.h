// Shared device/host helpers of libwvd (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wvd {

typedef uint16_t bf16_t;  // raw bf16 bits in memory

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

// bf16 -> fp32 is exact: the bf16 bits are the high half of the fp32 bits.
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN. gfx950 converts in hardware
// (v_cvt_pk_bf16_f32, two values per instruction), which the compiler emits for these conversions.
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float floatx2_t;
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const floatx2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// SiLU(v) = v * sigmoid(v) = v / (1 + e^-v), with the hardware exp2 and reciprocal.
__device__ __forceinline__ float silu_f32(float v) {
  const float e = __builtin_amdgcn_exp2f(-v * 1.4426950408889634f);
  return v * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace wvd

// Host-side launch helpers (defined in the .hip files, called by api.cpp).
namespace wvd {

// Side work of a kernel launch: up to two byte ranges copied (16-byte multiples, 16-byte
// aligned) that the kernel itself neither reads nor writes otherwise (the next history of a
// double-buffered cache slot). Each workgroup copies its share once its own work is done, so
// the copy runs beside other workgroups' matrix work.
struct CopyJob {
  const void* src[2];
  void* dst[2];
  int64_t bytes[2];
};

// The share of workgroup wg of nwg (threads tid of nthreads) of a CopyJob: 16-byte vector loads
// and stores, four in flight per thread.
__device__ __forceinline__ void run_copy_job(const CopyJob& c, int64_t wg, int64_t nwg, int tid, int nthreads) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = c.bytes[j] >> 4;
    if (n == 0) continue;
    const uint4* src = (const uint4*)c.src[j];
    uint4* dst = (uint4*)c.dst[j];
    const int64_t stride = nwg * nthreads;
    int64_t i = wg * nthreads + tid;
    for (; i + 3 * stride < n; i += 4 * stride) {
      const uint4 a = src[i], b = src[i + stride], d = src[i + 2 * stride], e = src[i + 3 * stride];
      dst[i] = a;
      dst[i + stride] = b;
      dst[i + 2 * stride] = d;
      dst[i + 3 * stride] = e;
    }
    for (; i < n; i += stride) dst[i] = src[i];
  }
}

// run_copy_job over the whole launch: this workgroup's share.
__device__ __forceinline__ void run_copy_share(const CopyJob& c) {
  const int64_t wg = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
  const int64_t nwg = (int64_t)gridDim.x * gridDim.y * gridDim.z;
  const int tid = threadIdx.x + blockDim.x * (threadIdx.y + blockDim.y * threadIdx.z);
  run_copy_job(c, wg, nwg, tid, blockDim.x * blockDim.y * blockDim.z);
}

// One convolution "problem" for the matrix-core implicit-GEMM kernel. The GEMM is
//   D[n][m] = sum_k Wpk[phase][n][k] * A[k][m]
// with m an output position of the input grid (t, h, w), n an output channel and k a (tap,
// input channel) pair. A[k][m] is the input element at the tap's offset from m, read from `x`
// (frames >= 0), `hist` (frames -Th..-1) or zero (outside the grid or before the history).
struct ConvProblem {
  const bf16_t* x;     // [T][H][W][Ci]
  const bf16_t* hist;  // [Th][H][W][Ci] or null
  int T, H, W, Ci, Th;
  const bf16_t* wpk;   // packed weights [phases][Npad][ntaps][Cip]
  int ntaps, Cip, Npad, phases;
  // Taps: with phases == 1, tap = (i*kh + j)*kw + k has offsets (i - 2*(kt/2), j - kh/2, k - kw/2);
  // with phases == 4 (x2 spatial upsampling), phase (a, b) tap u*2 + v has offsets
  // (0, u + a - 1, v + b - 1).
  int kt, kh, kw;
  int N;               // real output channels (columns stored)
  const float* bias;   // [N] or null
  // Output mapping: output element (n, t, h, w, phase p=(a,b)) goes to
  //   frame f = fbase + fmul*t + fstride*(n / nsplit), channel n % nsplit,
  //   row = hmul*h + a, col = wmul*w + b   (a = p / 2, b = p % 2 when phases == 4)
  // in y [To][Ho][Wo][nsplit] (NTHWC), bf16, or fp32 when y_f32 is set (channels n >= N of a
  // 4-channel group are then stored as zeros).
  void* y;
  const bf16_t* res;   // bf16 residual with y's layout and shape, or null (bf16 output only)
  int To, Ho, Wo, nsplit, fbase, fmul, fstride, hmul, wmul;
  int y_f32;
  // Optional fused channel RMS norm (+ SiLU) of the output (bf16 output, no residual, one
  // channel tile, see conv_can_fuse_norm): y = SiLU(gamma * v / sqrt(mean_c v^2 + eps)).
  const float* norm_gamma;  // [N] or null
  float norm_eps;
  int norm_silu;
  // With a fused norm, optionally also the pre-norm value (bias and residual added, one bf16
  // rounding) in y's layout: the residual stream beside the next block's activated input.
  bf16_t* y_pre;
  // With the dual store on the 192-channel x2 phase tile, the pre-norm value's 1x1 product in
  // place of the value itself (the next residual block's shortcut, that value's only reader):
  // y_sc = sc_w x bf16(pre-norm) + sc_b, fp32 sums, one rounding, in y's layout with sc_co
  // channels; sc_w row o holds output channel o's 192 weights at sc_w + o * sc_wrow.
  const bf16_t* sc_w;
  const float* sc_b;  // [sc_co] or null
  bf16_t* y_sc;
  int sc_co, sc_wrow;
  int time_tiles;  // set by the launcher: the halo kernel's tile order
  int staged;      // set by the launcher: store the output through LDS (see conv_epilogue_staged)
  CopyJob copy;    // side work (zero bytes: none)
  // The fused tail (head_w set): this x2 phase conv with norm_out + SiLU in its epilogue feeds the
  // output head (a causal 3x3x3 conv to head_co <= 3 colours) inside the same kernel, so the
  // activated tensor never reaches memory. head_w: the head's packed weight [Npad][3][Cip] (row
  // (j*3 + k)*4 + o, temporal tap, channel); head_b [head_co]; the video NCTHW bf16 with
  // video_frames frames per colour plane, this pass starting at frame video_fbase; carry
  // [2][3][2H][2W] fp32: the head's partial sums of the two frames after the pass (read when
  // carry_valid, written at the end).
  const bf16_t* head_w;
  const float* head_b;
  int head_co;
  bf16_t* video;
  int64_t video_frames;
  int video_fbase;
  float* carry;
  int carry_valid;
};

// force_config >= 0 runs that configuration (hipErrorNotSupported when it cannot run p);
// max_workgroups > 0 caps the workgroups of a DMA kernel launch, each then walking more tiles.
hipError_t launch_conv_mfma(const ConvProblem& p, hipStream_t s, int* config_id, int force_config = -1,
                            int max_workgroups = 0);
// Whether a conv with N output channels can apply RMS norm (+ SiLU) with gamma in its epilogue:
// one channel tile, N % 8 == 0, bias (may be null) and gamma 16-byte aligned.
bool conv_can_fuse_norm(int N, const float* bias, const float* gamma);
// The width condition alone (bias and gamma 16-byte aligned assumed).
bool conv_can_fuse_norm_width(int N);
const char* conv_config_name(int config_id);
int conv_config_count();

hipError_t launch_conv_fp32(const float* x, const float* hist, const float* w, const float* bias, float* y, int Ci,
                            int T, int H, int W, int Th, int Co, int kt, int kh, int kw, int layout_ncthw,
                            hipStream_t s);

// A residual block's norm1 + SiLU (act, [P][C]) and 1x1 shortcut (sc = W x + bias, [P][N]) from
// one read of x [P][C] (NTHWC bf16): C = 384, N a multiple of 32 up to 192, wpk the shortcut's
// packed weight (rows of C channels); both outputs equal the separate norm and 1x1 conv bit for bit.
bool norm_shortcut_supported(int C, int N);
hipError_t launch_norm_shortcut(const bf16_t* x, int64_t positions, int C, const float* gamma, float eps, bf16_t* act,
                                const bf16_t* wpk, int N, const float* bias, bf16_t* sc, hipStream_t s);
hipError_t launch_norm_silu(const bf16_t* x, const float* gamma, float eps, int silu, bf16_t* y, int64_t positions,
                            int C, hipStream_t s);

// The real topology's extra parts (topology.hip): the attention's row softmax (P = softmax of
// scale * S per row, bf16) and value transpose (vt [C][ldo] from v [R][C], zero columns R..ldo),
// the DupUp3D add (y [To][2H][2W][Co] += dup of x [T][H][W][Ci], output frame f + fo = ft*t + a),
// and unpatchify (+ clamp) of out [T][h][w][colours*patch^2] into the NCTHW video at fbase.
hipError_t launch_softmax_rows(const float* S, int64_t ld_s, int rows, int cols, float scale, bf16_t* P, int64_t ld_p,
                               hipStream_t s);
hipError_t launch_transpose_pad(const bf16_t* v, int R, int C, bf16_t* vt, int ldo, hipStream_t s);
hipError_t launch_dup_add(bf16_t* y, const bf16_t* x, int To, int T, int H, int W, int Ci, int Co, int ft, int fo,
                          hipStream_t s);
hipError_t launch_unpatchify(const bf16_t* out, int T, int h, int w, int colours, int patch, int clamp, bf16_t* video,
                             int64_t frames, int fbase, hipStream_t s);

hipError_t launch_convert(const void* x, int x_bf16, int x_ncthw, void* y, int y_bf16, int y_ncthw, int C, int T,
                          int H, int W, hipStream_t s);

// Pack raw weights [Co][Ci][kt][kh][kw] (fp32 or bf16) into [phases][Npad][ntaps][Cip] bf16.
hipError_t launch_pack_conv(const void* w, int w_bf16, int Co, int Ci, int ntaps_raw, int Npad, int Cip,
                            bf16_t* out, hipStream_t s);
hipError_t launch_pack_phase2x(const void* w, int w_bf16, int Co, int Ci, int Npad, int Cip, bf16_t* out,
                               hipStream_t s);
hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s);

// Output head (Co <= 4 output channels). Raw conv_out weight [Co][Ci][3][3][3] -> a temporal
// (3,1,1) conv with 36 outputs, output n = (j*3 + k)*4 + o taking W[o][:, :, j, k] (zero for o >= Co),
// packed [Npad][3][Cip] bf16.
hipError_t launch_pack_head(const void* w, int w_bf16, int Co, int Ci, int Npad, int Cip, bf16_t* out, hipStream_t s);
// video[o][fbase + t][h][w] = bias[o] + sum_{j,k} Z[j*3+k][t][h+j-1][w+k-1][o] (zero outside the frame),
// Z fp32 [9][T][H][W][4] tap planes; video bf16 NCTHW with `frames` frames per channel plane.
// The head's tap conv and stencil fused (input channels padded to Cip <= 192): x [T][H][W][C]
// bf16 with Th history frames, packed head weights [64][3][Cip], video NCTHW bf16.
bool head_fused_supported(int Cip);
// The input-stationary variant (each input frame read once per tile): Cip <= 96, Co <= 3; same
// arguments and output.
bool head_stream_supported(int Cip, int Co);
// Whether the fused tail (ConvProblem::head_w) takes an upsample of N channels (padded Cip) with a
// head of co colours: the 96-wide one-row phase tile, so 64 < N <= 96, N % 8 == 0, co <= 3.
bool tail_kernel_supported(int N, int Cip, int co);
// A device copy through the conv kernels' 16-byte buffer-load-to-LDS path (counter calibration).
hipError_t launch_dma_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);
// Winograd F(2x2, 3x3) steps (winograd.hip): the weight transform into 16 packed (3,1,1) weights,
// the input transform into U [16][Th+T][tH][tW][C] and the output transform of M [16][T][tH][tW][Co].
hipError_t launch_wino_pack(const void* w, int w_bf16, int Co, int Ci, int Npad, int Cip, bf16_t* out, hipStream_t s);
hipError_t launch_wino_in(const bf16_t* x, const bf16_t* hist, int T, int Th, int H, int W, int C, bf16_t* U,
                          hipStream_t s);
hipError_t launch_wino_out(const float* M, int T, int H, int W, int Co, const float* bias, const bf16_t* res,
                           bf16_t* y, hipStream_t s);
// The input-stationary head over T frames of x, its temporal taps from the frames before them
// carried in (cin: the partial sums left by the previous launch, or null for none) and out (cout,
// a different buffer of head_stream_carry_frame_bytes(H, W) * 2 bytes).
size_t head_stream_carry_frame_bytes(int H, int W);
hipError_t launch_head_stream(const bf16_t* x, int T, int H, int W, int C, int Cip, const bf16_t* wpk,
                              const float* bias, int Co, bf16_t* video, int64_t frames, int fbase, const float* cin,
                              float* cout, hipStream_t s);
hipError_t launch_head_fused(const bf16_t* x, const bf16_t* hist, int Th, int T, int H, int W, int C, int Cip,
                             const bf16_t* wpk, const float* bias, int Co, bf16_t* video, int64_t frames, int fbase,
                             hipStream_t s, const CopyJob* copy = nullptr);
hipError_t launch_head_stencil(const float* Z, int Co, const float* bias, bf16_t* video, int64_t frames, int fbase,
                               int T, int H, int W, hipStream_t s);

}  // namespace wvd
