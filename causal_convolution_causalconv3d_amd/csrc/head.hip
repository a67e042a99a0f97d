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

// Fused head: the tap conv and the stencil in one kernel, so the fp32 tap planes never go to
// memory. A workgroup computes Z (36 tap channels: tap*4 + colour) for a 16 x 32 tile of one
// frame that overlaps its neighbours by one pixel on every side, keeps Z in LDS, and sums the
// 9-tap stencil for the 14 x 30 interior straight into the video. Z at positions outside the
// frame is 0 (their activations read as 0), which is the conv's zero padding. Weights (64 rows:
// 36 used; 3 temporal taps x Cip channels) stay in LDS for the whole reduction, so the K loop has
// no barriers; the activation operands come from memory into registers through range-checked
// buffer loads, one K step ahead. The K order (32-channel chunk outermost, temporal tap inside,
// K halves in order) is the tap conv's, so Z is the same as the two-kernel path computes.
constexpr int HF_ROWS = 16, HF_COLS = 32;                      // computed tile
constexpr int HF_OROWS = HF_ROWS - 2, HF_OCOLS = HF_COLS - 2;   // output tile
constexpr int HF_N = 64;                                        // Z rows in the matrix-core tile
constexpr int HF_Z = 36;                                        // Z channels kept
constexpr int HF_MAXCIP = 192;
constexpr int HF_WROW = 3 * HF_MAXCIP + 8;  // bf16 per LDS weight row: 1168 bytes, 73 16-byte units (odd)
constexpr int HF_LDS = (HF_N * HF_WROW * 2 > HF_ROWS * HF_COLS * HF_Z * 4) ? HF_N * HF_WROW * 2
                                                                          : HF_ROWS * HF_COLS * HF_Z * 4;

__global__ __launch_bounds__(512, 1) void head_fused_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ hist,
                                                            int Th, int T, int H, int W, int C, int Cip,
                                                            const bf16_t* __restrict__ wpk, const float* __restrict__ bias,
                                                            int Co, bf16_t* __restrict__ video, int64_t frames, int fbase,
                                                            const CopyJob copy) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[HF_LDS];
  bf16_t* wl = (bf16_t*)lds;   // [64][HF_WROW] during the K loop
  float* zl = (float*)lds;     // [16][32][36] afterwards
  typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, l32 = lane & 31;
  const int numR = (H + HF_OROWS - 1) / HF_OROWS, numC = (W + HF_OCOLS - 1) / HF_OCOLS;
  const int total = T * numR * numC;
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int q8 = total >> 3, r8 = total & 7;
  const int lin = xcd * q8 + (xcd < r8 ? xcd : r8) + local;
  const int t = lin % T, tile = lin / T;  // time-fastest: a patch serves the temporal taps of neighbours
  const int rt = tile / numC;
  const int h0 = rt * HF_OROWS, w0 = (tile - rt * numC) * HF_OCOLS;  // first output pixel

  // weights into LDS: [n][i*Cip + c] from the packed [64][3][Cip]
  const int wk = 3 * Cip;
  for (int q = tid; q < HF_N * (wk / 8); q += 512) {
    const int n = q / (wk / 8), k8 = q - n * (wk / 8);
    *(u32x4*)(&wl[n * HF_WROW + k8 * 8]) = *(const u32x4*)(wpk + (int64_t)n * wk + k8 * 8);
  }

  // this lane's positions: tile rows 2*wave + mb (image row h0 - 1 + that), column l32
  const int64_t frame_elems = (int64_t)H * W * C;
  const uint32_t frame_bytes = (uint32_t)(frame_elems * 2);
  uint32_t poff[2];
  bool pin[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int hh = h0 - 1 + 2 * wave + mb, ww = w0 - 1 + l32;
    pin[mb] = (hh >= 0) & (hh < H) & (ww >= 0) & (ww < W);
    poff[mb] = pin[mb] ? (uint32_t)(((int64_t)hh * W + ww) * C * 2) : 0u;
  }
  const int nchunks = Cip >> 5;
  const int nk = 3 * nchunks;
  auto load_step = [&](u32x4 (&dst)[2][2], int s) {
    const int chunk = s / 3, i = s - chunk * 3;
    const int sf = t - 2 + i;  // source frame; negative: history
    const bf16_t* fb = (sf >= 0) ? x + (int64_t)sf * frame_elems
                                 : ((sf >= -Th) ? hist + (int64_t)(sf + Th) * frame_elems : x);
    const bool fok = (sf >= -Th) & (s < nk);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)fb, (short)0, fok ? (int)frame_bytes : 0, 0x00020000);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int ch = chunk * 32 + half * 16 + q * 8;
        const int vo = (pin[mb] & (ch < C)) ? (int)(poff[mb] + ch * 2) : (int)frame_bytes;
        dst[mb][q] = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, 0, 0);
      }
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.0f;

  u32x4 areg[2][2][2];
  load_step(areg[0], 0);
  __syncthreads();  // weights in place
  for (int s = 0; s < nk; s += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int st = s + u;
      load_step(areg[u ^ 1], st + 1);  // past the end: zeros, never used
      if (st < nk) {
        const int chunk = st / 3, i = st - chunk * 3;
        const int k0 = i * Cip + chunk * 32;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
              const u32x4 a = *(const u32x4*)(&wl[(nb * 32 + l32) * HF_WROW + k0 + half * 16 + q * 8]);
              acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                                    __builtin_bit_cast(bf16x8, areg[u][mb][q]),
                                                                    acc[nb][mb], 0, 0, 0);
            }
      }
    }
  }
  __syncthreads();  // every wave is done with the weights: the LDS now takes Z

  // Z[row][col][n] for n < 36 (lane: channels nb*32 + g*8 + half*4 + {0..3} of its position)
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    float* zp = zl + ((2 * wave + mb) * HF_COLS + l32) * HF_Z;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n = g * 8 + half * 4;
      *(float4*)(zp + n) = make_float4(acc[0][mb][g * 4], acc[0][mb][g * 4 + 1], acc[0][mb][g * 4 + 2],
                                       acc[0][mb][g * 4 + 3]);
    }
    if (half == 0) *(float4*)(zp + 32) = make_float4(acc[1][mb][0], acc[1][mb][1], acc[1][mb][2], acc[1][mb][3]);
  }
  __syncthreads();

  // the stencil: output pixel (h0 + orow, w0 + ocol) sums tap (j, k) of tile position
  // (orow + j, ocol + k); fp32 sums in (j, k) order, one rounding
  if (tid < HF_OROWS * HF_OCOLS) {
    const int orow = tid / HF_OCOLS, ocol = tid - orow * HF_OCOLS;
    const int h = h0 + orow, w = w0 + ocol;
    if (h < H && w < W) {
      float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
#pragma unroll
      for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          const float4 z = *(const float4*)(zl + ((orow + j) * HF_COLS + ocol + k) * HF_Z + (j * 3 + k) * 4);
          a0 += z.x;
          a1 += z.y;
          a2 += z.z;
          a3 += z.w;
        }
      const int64_t HW = (int64_t)H * W;
      const int64_t pix = (int64_t)(fbase + t) * HW + (int64_t)h * W + w;
      const float av[4] = {a0, a1, a2, a3};
#pragma unroll
      for (int o = 0; o < 4; ++o)
        if (o < Co) video[(int64_t)o * frames * HW + pix] = (bf16_t)f32_to_bf16(av[o] + (bias ? bias[o] : 0.0f));
    }
  }
  run_copy_share(copy);
}

// Input-stationary fused head (Cip <= 96, Co <= 3). A workgroup owns one 16 x 32 tile (14 x 30
// outputs, one-pixel overlap as above) and walks the frames: each input frame f is loaded once
// and feeds the three outputs it belongs to, Z_f (temporal tap 2), Z_{f+1} (tap 1) and Z_{f+2}
// (tap 0), whose accumulators rotate after every frame; Z_f is then complete and goes through
// LDS to the stencil. So the activations are read once per tile instead of once per temporal
// tap, and only the 27 tap channels in use (9 taps x 3 colours, one 32-row matrix block) are
// computed. The next frame's operands load into registers while the current one computes. The
// sum order of a Z value is temporal tap outermost, then chunk, then K half.
//
// The frames before the launch enter as a carry instead of as input frames: Z of the launch's
// output frames 0 and 1 as far as those earlier frames contribute (taps 0 and 1 of frame 0, tap
// 0 of frame 1), the two accumulators as they stood after the previous launch's last frame, in
// fp32. The launch starts its accumulators from them and leaves its own in `cout`, so a decode in
// several launches sums every Z value in the same order as one launch over all frames (same
// bits), reads no history frames and copies none. Carry layout, per buffer: [2 frames][7 planes]
// [H][W] float4, plane 2g + half holding rows 8g + 4 half + {0..3} of a position's Z column
// (rows 0-27; rows 28-31 have no weights and are always 0). Each tile reads the carry of all its
// 16 x 32 positions and writes that of its 14 x 30 interior (the tiles' interiors partition the
// frame), so `cin` and `cout` must be different buffers.
constexpr int HS_N = 27;  // tap rows kept: tap * 3 + colour
constexpr int HS_ZS = 28; // LDS floats per position for Z (27 + pad, 16-byte aligned rows)
constexpr int HS_CP = 7;  // carry planes (float4) per position and frame

template <int NCH>
__global__ __launch_bounds__(512, 1) void head_stream_kernel(const bf16_t* __restrict__ x, int T, int H, int W, int C,
                                                             const bf16_t* __restrict__ wpk, const float* __restrict__ bias,
                                                             int Co, bf16_t* __restrict__ video, int64_t frames, int fbase,
                                                             const float4* __restrict__ cin, float4* __restrict__ cout) {
  constexpr int Cip = NCH * 32;
  __shared__ __attribute__((aligned(16))) bf16_t wl[32 * HF_WROW];
  __shared__ __attribute__((aligned(16))) float zs[HF_ROWS * HF_COLS * HS_ZS];
  typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
  typedef float f32x4v __attribute__((ext_vector_type(4)));

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, l32 = lane & 31;
  const int numR = (H + HF_OROWS - 1) / HF_OROWS, numC = (W + HF_OCOLS - 1) / HF_OCOLS;
  const int total = numR * numC;
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int q8 = total >> 3, r8 = total & 7;
  const int lin = xcd * q8 + (xcd < r8 ? xcd : r8) + local;
  if (lin >= total) return;
  // Tiles in bands of HS_BAND tile rows, each band walked column by column: the workgroups an XCD
  // runs at once (a run of consecutive tiles) then cover a 2D block of the frame, so a tile's
  // halo rows and columns, which its neighbours above, below and beside read too, are read
  // from HBM about once while they sit in that XCD's L2 (in row order the neighbours below ran a
  // round later, after the rows had left L2).
  constexpr int HS_BAND = 4;
  const int band = lin / (HS_BAND * numC);
  const int r0 = band * HS_BAND, bh = (numR - r0 < HS_BAND) ? numR - r0 : HS_BAND;
  const int bidx = lin - band * HS_BAND * numC;
  const int rt = r0 + bidx % bh, ct = bidx / bh;
  const int h0 = rt * HF_OROWS, w0 = ct * HF_OCOLS;

  // weights into LDS: row n = tap * 3 + o of the 32-row block from packed row tap * 4 + o
  constexpr int WK8 = 3 * Cip / 8;
  for (int q = tid; q < 32 * WK8; q += 512) {
    const int n = q / WK8, k8 = q - n * WK8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n < HS_N) v = *(const u32x4*)(wpk + (int64_t)((n / 3) * 4 + n % 3) * (3 * Cip) + k8 * 8);
    *(u32x4*)(&wl[n * HF_WROW + k8 * 8]) = v;
  }

  // this lane's positions: tile rows 2*wave + mb (image row h0 - 1 + that), column l32
  const int64_t frame_elems = (int64_t)H * W * C;
  const int HW = H * W;  // (< 2^30: a frame of C >= 1 channels is under 2^31 bytes)
  const uint32_t frame_bytes = (uint32_t)(frame_elems * 2);
  uint32_t poff[2];
  bool pin[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int hh = h0 - 1 + 2 * wave + mb, ww = w0 - 1 + l32;
    pin[mb] = (hh >= 0) & (hh < H) & (ww >= 0) & (ww < W);
    poff[mb] = pin[mb] ? (uint32_t)((hh * W + ww) * C * 2) : 0u;
  }
  // carry index of this lane's position of tile row 2*wave + mb (frame 0, plane 0)
  auto cpos = [&](int mb) { return (h0 - 1 + 2 * wave + mb) * W + (w0 - 1 + l32); };
  // the operands of frame f, all chunks
  auto load_frame = [&](u32x4 (&dst)[NCH][2][2], int f) {
    const bf16_t* fb = x + (int64_t)f * frame_elems;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)fb, (short)0, (int)frame_bytes, 0x00020000);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int ch = c * 32 + half * 16 + q * 8;
          const int vo = (pin[mb] & (ch < C)) ? (int)(poff[mb] + ch * 2) : (int)frame_bytes;
          dst[c][mb][q] = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, 0, 0);
        }
  };

  u32x4 breg[2][NCH][2][2];
  load_frame(breg[0], 0);

  // Z_f, Z_{f+1}, Z_{f+2} while frame f is consumed; Z_0 and Z_1 start from the carry
  floatx16 za[2], zb[2], zc[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int pl = 2 * g + half;
      float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f), c = a;
      if (cin && pin[mb] && pl < HS_CP) {
        a = cin[pl * HW + cpos(mb)];
        c = cin[(HS_CP + pl) * HW + cpos(mb)];
      }
      za[mb][g * 4 + 0] = a.x;
      za[mb][g * 4 + 1] = a.y;
      za[mb][g * 4 + 2] = a.z;
      za[mb][g * 4 + 3] = a.w;
      zb[mb][g * 4 + 0] = c.x;
      zb[mb][g * 4 + 1] = c.y;
      zb[mb][g * 4 + 2] = c.z;
      zb[mb][g * 4 + 3] = c.w;
#pragma unroll
      for (int e = 0; e < 4; ++e) zc[mb][g * 4 + e] = 0.0f;
    }
  // frame f's contributions: tap 0 to Z_{f+2}, tap 1 to Z_{f+1}, tap 2 to Z_f
  auto consume = [&](const u32x4 (&bf)[NCH][2][2]) {
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const u32x4 a0 = *(const u32x4*)(&wl[l32 * HF_WROW + 0 * Cip + c * 32 + half * 16 + q * 8]);
        const u32x4 a1 = *(const u32x4*)(&wl[l32 * HF_WROW + 1 * Cip + c * 32 + half * 16 + q * 8]);
        const u32x4 a2 = *(const u32x4*)(&wl[l32 * HF_WROW + 2 * Cip + c * 32 + half * 16 + q * 8]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8 bv = __builtin_bit_cast(bf16x8, bf[c][mb][q]);
          zc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a0), bv, zc[mb], 0, 0, 0);
          zb[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a1), bv, zb[mb], 0, 0, 0);
          za[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a2), bv, za[mb], 0, 0, 0);
        }
      }
  };
  // the carry of the next launch (after the last frame): Z of its frames 0 and 1 so far, at this
  // tile's interior positions (tile rows 1 .. 14, columns 1 .. 30); streamed out past the L2,
  // since the next read comes after a whole upsample launch
  auto store_carry = [&]() {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int trow = 2 * wave + mb;
      if (!(pin[mb] & (trow >= 1) & (trow <= HF_OROWS) & (l32 >= 1) & (l32 <= HF_OCOLS))) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int pl = 2 * g + half;
        if (pl >= HS_CP) continue;
        const f32x4v a = {za[mb][g * 4 + 0], za[mb][g * 4 + 1], za[mb][g * 4 + 2], za[mb][g * 4 + 3]};
        const f32x4v c = {zb[mb][g * 4 + 0], zb[mb][g * 4 + 1], zb[mb][g * 4 + 2], zb[mb][g * 4 + 3]};
        __builtin_nontemporal_store(a, (f32x4v*)(cout + pl * HW + cpos(mb)));
        __builtin_nontemporal_store(c, (f32x4v*)(cout + (HS_CP + pl) * HW + cpos(mb)));
      }
    }
  };
  float bo[3];
#pragma unroll
  for (int o = 0; o < 3; ++o) bo[o] = (bias && o < Co) ? bias[o] : 0.0f;
  // Z_t (in za) through LDS to the stencil, then the rotation
  auto finish = [&](int t) {
    __syncthreads();  // the previous frame's stencil is done with zs
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      float* zp = zs + ((2 * wave + mb) * HF_COLS + l32) * HS_ZS;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = g * 8 + half * 4;
        if (n < HS_N)
          *(float4*)(zp + n) = make_float4(za[mb][g * 4], za[mb][g * 4 + 1], za[mb][g * 4 + 2], za[mb][g * 4 + 3]);
      }
    }
    __syncthreads();
    if (tid < HF_OROWS * HF_OCOLS) {
      const int orow = tid / HF_OCOLS, ocol = tid - orow * HF_OCOLS;
      const int h = h0 + orow, w = w0 + ocol;
      if (h < H && w < W) {
        float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f;
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
          for (int k = 0; k < 3; ++k) {
            const float* z = zs + ((orow + j) * HF_COLS + ocol + k) * HS_ZS + (j * 3 + k) * 3;
            a0 += z[0];
            a1 += z[1];
            a2 += z[2];
          }
        const int64_t pix = (int64_t)(fbase + t) * HW + h * W + w;
        const float av[3] = {a0, a1, a2};
#pragma unroll
        for (int o = 0; o < 3; ++o)
          if (o < Co) video[(int64_t)o * frames * HW + pix] = (bf16_t)f32_to_bf16(av[o] + bo[o]);
      }
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      za[mb] = zb[mb];
      zb[mb] = zc[mb];
#pragma unroll
      for (int r = 0; r < 16; ++r) zc[mb][r] = 0.0f;
    }
  };

  __syncthreads();  // weights in place
  // frames in pairs while a frame follows the pair, then the last one or two: the loop has one
  // exit, so the accumulators leave it in fixed registers for the carry's stores
  int f = 0;
  for (; f + 2 < T; f += 2) {
    load_frame(breg[1], f + 1);
    consume(breg[0]);
    finish(f);
    load_frame(breg[0], f + 2);
    consume(breg[1]);
    finish(f + 1);
  }
  if (f + 1 < T) {
    load_frame(breg[1], f + 1);
    consume(breg[0]);
    finish(f);
    consume(breg[1]);
    finish(f + 1);
  } else {
    consume(breg[0]);
    finish(f);
  }
  store_carry();
}

}  // namespace

hipError_t launch_pack_head(const void* w, int w_bf16, int Co, int Ci, int Npad, int Cip, bf16_t* out, hipStream_t s) {
  const int64_t n = (int64_t)Npad * 3 * Cip;
  hipLaunchKernelGGL(pack_head_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, w, w_bf16, Co, Ci, Npad,
                     Cip, out);
  return hipGetLastError();
}

bool head_fused_supported(int Cip) { return Cip % 32 == 0 && Cip <= HF_MAXCIP; }

bool head_stream_supported(int Cip, int Co) { return Cip % 32 == 0 && Cip <= 96 && Co <= 3; }

size_t head_stream_carry_frame_bytes(int H, int W) { return (size_t)H * W * HS_CP * 16; }

hipError_t launch_head_stream(const bf16_t* x, int T, int H, int W, int C, int Cip, const bf16_t* wpk,
                              const float* bias, int Co, bf16_t* video, int64_t frames, int fbase, const float* cin,
                              float* cout, hipStream_t s) {
  if (T == 0 || H == 0 || W == 0) return hipSuccess;
  // (the kernel indexes a frame's bytes and the carry's float4 planes, 2 x 7 per position, in 32 bits)
  if (!head_stream_supported(Cip, Co) || C > Cip || (int64_t)H * W * C * 2 >= ((int64_t)1 << 31) ||
      (int64_t)H * W * 2 * HS_CP >= ((int64_t)1 << 31) || !cout || cout == cin || ((uintptr_t)cin & 15u) ||
      ((uintptr_t)cout & 15u))
    return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)((H + HF_OROWS - 1) / HF_OROWS) * ((W + HF_OCOLS - 1) / HF_OCOLS);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const float4* ci = (const float4*)cin;
  float4* co = (float4*)cout;
  switch (Cip / 32) {
    case 1:
      hipLaunchKernelGGL(head_stream_kernel<1>, dim3((unsigned)blocks), dim3(512), 0, s, x, T, H, W, C, wpk, bias, Co,
                         video, frames, fbase, ci, co);
      break;
    case 2:
      hipLaunchKernelGGL(head_stream_kernel<2>, dim3((unsigned)blocks), dim3(512), 0, s, x, T, H, W, C, wpk, bias, Co,
                         video, frames, fbase, ci, co);
      break;
    default:
      hipLaunchKernelGGL(head_stream_kernel<3>, dim3((unsigned)blocks), dim3(512), 0, s, x, T, H, W, C, wpk, bias, Co,
                         video, frames, fbase, ci, co);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_head_fused(const bf16_t* x, const bf16_t* hist, int Th, int T, int H, int W, int C, int Cip,
                             const bf16_t* wpk, const float* bias, int Co, bf16_t* video, int64_t frames, int fbase,
                             hipStream_t s, const CopyJob* copy) {
  const CopyJob job = copy ? *copy : CopyJob{};
  if (T == 0 || H == 0 || W == 0) return hipSuccess;
  if (!head_fused_supported(Cip) || C > Cip || (int64_t)H * W * C * 2 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)T * ((H + HF_OROWS - 1) / HF_OROWS) * ((W + HF_OCOLS - 1) / HF_OCOLS);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(head_fused_kernel, dim3((unsigned)blocks), dim3(512), 0, s, x, hist, Th, T, H, W, C, Cip, wpk, bias,
                     Co, video, frames, fbase, job);
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
