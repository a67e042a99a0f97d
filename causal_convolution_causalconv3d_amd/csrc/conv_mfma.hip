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
#include <type_traits>

#include "conv_epilogue.h"

namespace wvd {

namespace {

constexpr int LDS_ROW = 40;  // bf16 per LDS row: 32 channels + 8 pad (80 bytes: no bank conflicts)

// Staging pieces are 16 bytes (8 channels of one weight row or patch position), four lanes per
// row so that a wave's global loads cover whole 64-byte runs. A lane without a piece (the last
// round of a tile whose piece count is not a multiple of the workgroup size) loads a valid
// address and stores into the unused 16-byte pad of a row, one pad per such lane: no branch,
// and no pile-up of many lanes on one LDS address (a same-address store serialises).
__device__ __forceinline__ int pad_slot(int row) { return row * LDS_ROW + 32; }  // in bf16

template <int NB, int MB, int WAVES, bool NORM>
__global__ __launch_bounds__(WAVES * 64, 1) void conv_mfma_kernel(const ConvProblem p) {
  constexpr int BN = NB * 32;
  constexpr int BM = WAVES * MB * 32;
  constexpr int NT = WAVES * 64;
  constexpr int WPIECES = BN * 4;  // 16-byte pieces of one weight K step
  constexpr int WLOADS = (WPIECES + NT - 1) / NT;
  // weight stages; after the K loop, the per-wave areas of the staged epilogue (one-block waves)
  constexpr int NBPL = (NB % 3 == 0) ? 3 : ((NB % 2 == 0) ? 2 : 1);
  constexpr int SBL = StagedShape<NBPL>::BYTES;
  constexpr int LDS_ELEMS = (MB == 1 && WAVES * SBL / 2 > 4 * BN * LDS_ROW) ? WAVES * SBL / 2 : 4 * BN * LDS_ROW;
  __shared__ __attribute__((aligned(16))) bf16_t lds_all[LDS_ELEMS];
  bf16_t(*lds)[BN * LDS_ROW] = reinterpret_cast<bf16_t(*)[BN * LDS_ROW]>(lds_all);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int phase = blockIdx.z;

  const int HW = p.H * p.W;
  // M tiles never straddle a frame, so the source frame of every tap is uniform per workgroup.
  const int tpf = (HW + BM - 1) / BM;  // tiles per frame
  const int numM = p.T * tpf;
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
  // Tile order: a conv with spatial taps runs a frame's tiles next to each other (neighbouring
  // rows meet in L2); a temporal-only conv (the time upsample, the head) runs the same positions
  // of consecutive frames next to each other, so its three temporal taps hit in L2.
  const bool time_fast = (p.kh == 1) & (p.kw == 1) & (p.phases == 1);
  const int tf = time_fast ? mt % p.T : mt / tpf;                  // the tile's frame
  const int tile = time_fast ? mt / p.T : mt - tf * tpf;
  const int mbase = tile * BM + wave * (MB * 32);                  // position within the frame

  const int pa = (p.phases == 4) ? (phase >> 1) : 0;
  const int pb = (p.phases == 4) ? (phase & 1) : 0;
  // tap offsets: (i - 2*(kt/2), j - kh/2, k - kw/2), or for a phase (0, j + a - 1, k + b - 1)
  const int dt0 = (p.phases == 4) ? 0 : -2 * (p.kt >> 1);
  const int dh0 = (p.phases == 4) ? pa - 1 : -(p.kh >> 1);
  const int dw0 = (p.phases == 4) ? pb - 1 : -(p.kw >> 1);

  // Per lane and row block: the position (h, w), its byte offset in a frame, and a mask of the
  // spatial taps (j, k) whose neighbour lies inside the frame (bit j*kw + k).
  int ph[MB], pw[MB];
  bool pv[MB];
  uint32_t loff[MB], smask[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = mbase + mb * 32 + l32;
    pv[mb] = m < HW;
    const int mm = pv[mb] ? m : 0;
    const int h = mm / p.W;
    const int w = mm - h * p.W;
    ph[mb] = h;
    pw[mb] = w;
    loff[mb] = (uint32_t)((mm * p.Ci + half * 16) * 2);
    uint32_t msk = 0;
    for (int j = 0; j < p.kh; ++j)
      for (int k = 0; k < p.kw; ++k) {
        const int hh = h + dh0 + j, ww = w + dw0 + k;
        if (pv[mb] && hh >= 0 && hh < p.H && ww >= 0 && ww < p.W) msk |= 1u << (j * p.kw + k);
      }
    smask[mb] = msk;
  }

  const int nchunks = p.Cip >> 5;
  const int nk = p.ntaps * nchunks;
  const int64_t frame_elems = (int64_t)HW * p.Ci;
  const uint32_t frame_bytes = (uint32_t)(frame_elems * 2);
  const int64_t wrow = (int64_t)p.ntaps * p.Cip;
  const bf16_t* wbase = p.wpk + ((int64_t)phase * p.Npad + n0) * wrow;

  typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
  u32x4 areg[3][MB][2];     // activations of steps k (in use), k + 1 and k + 2 (in flight)
  u32x4 wreg[2][WLOADS];    // weights of steps k + 2 and k + 3 on their way to LDS
  u32x4 wf[2][2][NB];       // weight fragments of steps k (in use) and k + 1 (read from LDS)

  // K order: the 32-channel chunk outermost, the taps inside it (k fastest), so consecutive K steps
  // read the same channels one position apart and mostly hit the L1 cache. The step count is
  // rounded up to a multiple of 6 (the register rotation period); cursors move without branches,
  // stop at the last real step, and activation loads of the padding steps return zeros, so those
  // steps add nothing.
  const int nk6 = (nk + 5) / 6 * 6;
  struct Cursor {
    int step, chunk, tap, ti, tj, tk;
  };
  auto advance = [&](Cursor& c) {
    const bool go = c.step + 1 < nk;
    const int tk1 = c.tk + 1;
    const bool wk = tk1 == p.kw;
    const int tj1 = c.tj + (wk ? 1 : 0);
    const bool wj = tj1 == p.kh;
    const int ti1 = c.ti + (wj ? 1 : 0);
    const bool wi = ti1 == p.kt;
    c.tk = go ? (wk ? 0 : tk1) : c.tk;
    c.tj = go ? (wj ? 0 : tj1) : c.tj;
    c.ti = go ? (wi ? 0 : ti1) : c.ti;
    c.chunk = go ? c.chunk + (wi ? 1 : 0) : c.chunk;
    c.tap = go ? (wi ? 0 : c.tap + 1) : c.tap;
    c.step = c.step + 1;  // keeps counting: steps >= nk are padding
  };
  // Activation operands come from range-checked buffer loads over one frame: the frame (current
  // input or history) is uniform, a lane whose tap falls outside the frame, before the history,
  // past the channels or in a padding step gets the out-of-range offset `frame_bytes` and the
  // hardware returns 0.
  auto load_act = [&](u32x4 (&dst)[MB][2], const Cursor& c) {
    const int s = tf + dt0 + c.ti;  // source frame (negative: history)
    const bool fok = (s >= -p.Th) & (c.step < nk);
    const bf16_t* fbase = (s >= 0) ? p.x + (int64_t)s * frame_elems
                                   : ((s >= -p.Th) ? p.hist + (int64_t)(s + p.Th) * frame_elems : p.x);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)fbase, (short)0, (int)frame_bytes, 0x00020000);
    const int uoff = (((dh0 + c.tj) * p.W + (dw0 + c.tk)) * p.Ci + c.chunk * 32) * 2;
    const int bit = c.tj * p.kw + c.tk;
    const int ch = c.chunk * 32 + half * 16;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const bool ok = fok & (((smask[mb] >> bit) & 1u) != 0u);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const bool use = ok & (ch + q * 8 < p.Ci);
        const int vo = use ? (int)loff[mb] + uoff + q * 16 : (int)frame_bytes;
        dst[mb][q] = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, 0, 0);
      }
    }
  };
  // Weight rows past Npad (only in a partial last N tile) read row Npad-1: those columns are
  // never stored. Lanes past the tile's pieces go to pad slots (see pad_slot).
  auto load_w = [&](u32x4 (&dst)[WLOADS], const Cursor& c) {
#pragma unroll
    for (int i = 0; i < WLOADS; ++i) {
      const int q = (tid + i * NT) % WPIECES;
      const int row = min(q >> 2, p.Npad - 1 - n0), piece = q & 3;
      dst[i] = *(const u32x4*)(wbase + row * wrow + c.tap * p.Cip + c.chunk * 32 + piece * 8);
    }
  };
  auto store_w = [&](const u32x4 (&src)[WLOADS], int buf) {
#pragma unroll
    for (int i = 0; i < WLOADS; ++i) {
      const int q = tid + i * NT;
      const int at = q < WPIECES ? (q >> 2) * LDS_ROW + (q & 3) * 8 : pad_slot((q - WPIECES) % BN);
      *(u32x4*)(&lds[buf][at]) = src[i];
    }
  };
  auto read_w = [&](u32x4 (&dst)[2][NB], int buf) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        dst[q][nb] = *(const u32x4*)(&lds[buf][(nb * 32 + l32) * LDS_ROW + half * 16 + q * 8]);
  };

  floatx16 acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.0f;

  auto compute = [&](const u32x4 (&a)[MB][2], const u32x4 (&w)[2][NB]) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w[q][nb]),
                                                                __builtin_bit_cast(bf16x8, a[mb][q]), acc[nb][mb],
                                                                0, 0, 0);
  };

  // Pipeline (LDS weight stages: step j in stage j % 4). Step k multiplies the activations loaded
  // during step k - 2 with the weight fragments read from LDS during step k - 1. Meanwhile it
  // loads the activations of step k + 2 and the weights of step k + 3 (into registers), reads the
  // fragments of step k + 1, and at its end stores the weights of step k + 2 (loaded during step
  // k - 1) into their LDS stage, which every wave finished reading three barriers earlier. Every
  // load has about two steps of matrix work to arrive.
  Cursor ca = {0, 0, 0, 0, 0, 0};  // activations: the next step to load
  Cursor cw = {0, 0, 0, 0, 0, 0};  // weights: the next step to load
  load_w(wreg[0], cw);
  advance(cw);
  store_w(wreg[0], 0);
  load_w(wreg[0], cw);
  advance(cw);
  store_w(wreg[0], 1);
  load_w(wreg[1], cw);  // step 2, stored at the end of step 0
  advance(cw);
  load_act(areg[0], ca);
  advance(ca);
  load_act(areg[1], ca);
  advance(ca);
  __syncthreads();
  read_w(wf[0], 0);

  constexpr int NMFMA = 2 * MB * NB;
  auto step = [&](auto S, int k) {
    constexpr int s6 = decltype(S)::value;
    constexpr int a_cur = s6 % 3, a_new = (s6 + 2) % 3;
    constexpr int w_new = s6 & 1, w_old = (s6 + 1) & 1;
    constexpr int f_cur = s6 & 1, f_new = (s6 + 1) & 1;
    load_w(wreg[w_new], cw);  // step k + 3
    advance(cw);
    load_act(areg[a_new], ca);  // step k + 2
    advance(ca);
    read_w(wf[f_new], (k + 1) & 3);
    compute(areg[a_cur], wf[f_cur]);
    // one matrix instruction, then a few others: VMEM loads first, LDS reads next
#pragma unroll
    for (int i = 0; i < NMFMA; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < WLOADS + 2 * MB) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      else if (i < WLOADS + 2 * MB + 2 * NB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x006, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    store_w(wreg[w_old], (k + 2) & 3);  // step k + 2
    __syncthreads();
  };
  for (int k = 0; k < nk6; k += 6) {
    step(std::integral_constant<int, 0>{}, k);
    step(std::integral_constant<int, 1>{}, k + 1);
    step(std::integral_constant<int, 2>{}, k + 2);
    step(std::integral_constant<int, 3>{}, k + 3);
    step(std::integral_constant<int, 4>{}, k + 4);
    step(std::integral_constant<int, 5>{}, k + 5);
  }

  if constexpr (MB == 1 && !NORM) {
    if (p.staged) {
      // The launcher sets staged only for the plain output mapping, where a wave's 32 positions
      // (consecutive in the frame) are consecutive in the output: the frame is staged as one
      // row of H*W columns. Every wave is past the loop's last barrier, so the weight stages
      // are free.
      ConvProblem q = p;
      q.H = 1;
      q.W = HW;
      q.Ho = 1;
      q.Wo = HW;
      const int row0[1] = {0};
      conv_epilogue_staged<NB, 1, false, NBPL>(q, acc, row0, mbase, tf, n0, 0, 0, lane,
                                               (char*)lds_all + wave * SBL);
      run_copy_share(p.copy);
      return;
    }
  }
  conv_epilogue<NB, MB, NORM>(p, acc, ph, pw, pv, tf, n0, pa, pb, half);
  run_copy_share(p.copy);
}

// Halo-tile variant for KS x KS spatial taps: KS = 3 (phases == 1, kh == kw == 3, any kt) or
// KS = 2 (the four 2x2 phase convs of the x2 upsampling, phases == 4, one workgroup per phase).
// A workgroup owns TR = WAVES*MB rows x 32 columns of one frame and BN = 32*NB output channels;
// wave w owns rows w*MB .. w*MB + MB - 1 (one 32-position block per row). The K loop runs over
// stages (32-channel chunk outermost, temporal tap inside), KS*KS steps (the spatial taps) per
// stage. A stage's input patch, (TR + 2) x 34 positions x 32 channels of the tap's source frame
// (the tile with a 1-pixel halo), is read from memory once, staged in LDS (double-buffered,
// 80-byte position stride: conflict-free 16-byte reads of 32 consecutive positions), and every
// spatial tap reads its activation operand from it. Out-of-frame, out-of-channel and
// pre-history reads are hardware zeros as above. The weights go through LDS one K step at a time
// as in conv_mfma_kernel.
constexpr int PROW = 40;  // bf16 per patch position: 32 channels + 8 pad

template <int NB, int MB, int WAVES, int KS, bool NORM>
__global__ __launch_bounds__(WAVES * 64, 8 / WAVES) void conv_halo_kernel(const ConvProblem p) {
  static_assert(KS == 2 || KS == 3, "3x3 taps, or 2x2 phase taps");
  constexpr int SPS = KS * KS;              // steps per stage
  constexpr int STORE_S = SPS == 9 ? 4 : 2;  // the step that stores the next stage's patch
  constexpr int BN = NB * 32;
  constexpr int TR = WAVES * MB;
  constexpr int PR = TR + 2, PC = 34;
  constexpr int PATCH = PR * PC * PROW;
  constexpr int NT = WAVES * 64;
  constexpr int WPIECES = BN * 4;
  constexpr int WLOADS = (WPIECES + NT - 1) / NT;
  constexpr int PPIECES = PR * PC * 4;  // 16-byte pieces of one patch
  constexpr int PLOADS = (PPIECES + NT - 1) / NT;
  static_assert(NT % 4 == 0, "a thread's pieces share one channel group");
  static_assert(PLOADS * NT - PPIECES <= PR * PC, "a pad slot for every lane without a patch piece");
  // Weight stages: step j's slice sits in stage j % NWS. Three suffice (stage (k + 2) % 3 is
  // written at the end of step k; its last reader, step k - 1, is past the barrier of step
  // k - 1); with 9 steps per stage the index is then a compile-time constant. 2x2 taps (4 steps
  // per stage) use four for the same reason.
  constexpr int NWS = (SPS % 3 == 0) ? 3 : 4;
  __shared__ __attribute__((aligned(16))) bf16_t lds_w[NWS][BN * LDS_ROW];
  __shared__ __attribute__((aligned(16))) bf16_t lds_p[2][PATCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int phase = blockIdx.z;
  const int pa = (KS == 2) ? (phase >> 1) : 0;
  const int pb = (KS == 2) ? (phase & 1) : 0;

  const int numR = (p.H + TR - 1) / TR, numC = (p.W + 31) / 32;
  const int tpf = numR * numC;
  const int numN = (p.Npad + BN - 1) / BN;
  const int total = p.T * tpf * numN;
  // XCD-aware order as in conv_mfma_kernel; the channel tiles of a position tile are adjacent
  // (they read the same patches).
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int q8 = total >> 3, r8 = total & 7;
  const int lin = xcd * q8 + (xcd < r8 ? xcd : r8) + local;
  const int mt = lin / numN, nt = lin - (lin / numN) * numN;
  const int n0 = nt * BN;
  // Tile order: frame-major (a frame's tiles next to each other), or with time_tiles the same
  // tile of consecutive frames next to each other (an input patch then serves the temporal taps
  // of three neighbouring workgroups while it is in L2).
  const int tf = p.time_tiles ? mt % p.T : mt / tpf;
  const int rem = p.time_tiles ? mt / p.T : mt - tf * tpf;
  const int rt = rem / numC;
  const int h0 = rt * TR, w0 = (rem - rt * numC) * 32;
  const int dt0 = -2 * (p.kt >> 1);

  int ph[MB], pw[MB];
  bool pv[MB];
  // Byte offset of this lane's operand for tap (0, 0) in a patch buffer: patch position
  // (r + 1 + dh0, l32 + 1 + dw0) with the first tap's offset (dh0, dw0) = (-1, -1), or for phase
  // (a, b) of the x2 upsampling (a - 1, b - 1).
  uint32_t boff[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = wave * MB + mb;
    ph[mb] = h0 + r;
    pw[mb] = w0 + l32;
    pv[mb] = (ph[mb] < p.H) & (pw[mb] < p.W);
    boff[mb] = (uint32_t)((((r + pa) * PC + l32 + pb) * PROW + half * 16) * 2);
  }

  // This thread's patch pieces: position (piece / 4) of the patch, channel group tid & 3; a lane
  // without a piece loads zeros and stores into a position's unused pad.
  const int ch8 = (tid & 3) * 8;
  int goff[PLOADS];       // byte offset in a frame (chunk 0), or -1 outside the frame
  uint32_t poff[PLOADS];  // byte offset in a patch buffer
#pragma unroll
  for (int i = 0; i < PLOADS; ++i) {
    const int piece = tid + i * NT;
    const int pos = piece >> 2;
    const int pr = pos / PC, pc = pos - (pos / PC) * PC;
    const int hh = h0 - 1 + pr, ww = w0 - 1 + pc;
    const bool inb = (piece < PPIECES) & (hh >= 0) & (hh < p.H) & (ww >= 0) & (ww < p.W);
    goff[i] = inb ? ((hh * p.W + ww) * p.Ci + ch8) * 2 : -1;
    poff[i] = (uint32_t)((piece < PPIECES ? pos * PROW + ch8 : pad_slot(piece - PPIECES)) * 2);
  }

  const int nchunks = p.Cip >> 5;
  const int ng = nchunks * p.kt;
  const int64_t frame_elems = (int64_t)p.H * p.W * p.Ci;
  const uint32_t frame_bytes = (uint32_t)(frame_elems * 2);
  const int64_t wrow = (int64_t)p.ntaps * p.Cip;
  const bf16_t* wbase = p.wpk + ((int64_t)phase * p.Npad + n0) * wrow;

  typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
  u32x4 wreg[2][WLOADS];  // weights of steps k + 2 and k + 3 on their way to LDS
  u32x4 preg[PLOADS];     // the next stage's patch on its way to LDS
  u32x4 wf[2][NB];        // weight fragments of the current and the next half step
  u32x4 bf[2][MB];        // activation fragments of the current and the next half step

  // Stage cursor: (chunk, temporal tap) of a stage and its weight column base.
  struct Stage {
    int chunk, i, col;
  };
  auto stage_at = [&](int chunk, int i) -> Stage { return {chunk, i, i * SPS * p.Cip + chunk * 32}; };
  auto next_stage = [&](const Stage& c) -> Stage {
    // past the last stage the cursor stays put (its loads are never used)
    if (c.chunk * p.kt + c.i + 1 >= ng) return c;
    return (c.i + 1 == p.kt) ? stage_at(c.chunk + 1, 0) : stage_at(c.chunk, c.i + 1);
  };

  auto load_patch = [&](u32x4 (&dst)[PLOADS], const Stage& c, bool live) {
    const int sf = tf + dt0 + c.i;  // source frame (negative: history)
    const bool fok = live & (sf >= -p.Th) & (c.chunk * 32 + ch8 < p.Ci);
    const bf16_t* fbase = (sf >= 0) ? p.x + (int64_t)sf * frame_elems
                                    : ((sf >= -p.Th) ? p.hist + (int64_t)(sf + p.Th) * frame_elems : p.x);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)fbase, (short)0, (int)frame_bytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < PLOADS; ++i) {
      const int vo = (fok & (goff[i] >= 0)) ? goff[i] + c.chunk * 64 : (int)frame_bytes;
      dst[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, 0, 0);
    }
  };
  auto store_patch = [&](const u32x4 (&src)[PLOADS], int buf) {
#pragma unroll
    for (int i = 0; i < PLOADS; ++i) *(u32x4*)((char*)lds_p[buf] + poff[i]) = src[i];
  };
  auto load_w = [&](u32x4 (&dst)[WLOADS], int col) {
#pragma unroll
    for (int i = 0; i < WLOADS; ++i) {
      const int q = (tid + i * NT) % WPIECES;
      const int row = min(q >> 2, p.Npad - 1 - n0), piece = q & 3;
      dst[i] = *(const u32x4*)(wbase + row * wrow + col + piece * 8);
    }
  };
  auto store_w = [&](const u32x4 (&src)[WLOADS], int buf) {
#pragma unroll
    for (int i = 0; i < WLOADS; ++i) {
      const int q = tid + i * NT;
      const int at = q < WPIECES ? (q >> 2) * LDS_ROW + (q & 3) * 8 : pad_slot((q - WPIECES) % BN);
      *(u32x4*)(&lds_w[buf][at]) = src[i];
    }
  };
  // fragments of K half q (channels half*16 + q*8 .. + 7 of the chunk) of spatial tap `tap`
  auto read_a = [&](u32x4 (&dst)[NB], int buf, int q) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) dst[nb] = *(const u32x4*)(&lds_w[buf][(nb * 32 + l32) * LDS_ROW + half * 16 + q * 8]);
  };
  auto read_b = [&](u32x4 (&dst)[MB], int buf, int tap, int q) {
    const int j = tap / KS, k = tap - (tap / KS) * KS;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      dst[mb] = *(const u32x4*)((const char*)lds_p[buf] + boff[mb] + ((j * PC + k) * PROW + q * 8) * 2);
  };

  floatx16 acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.0f;

  auto compute = [&](const u32x4 (&w)[NB], const u32x4 (&a)[MB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w[nb]),
                                                              __builtin_bit_cast(bf16x8, a[mb]), acc[nb][mb], 0, 0, 0);
  };

  // Pipeline. Weights: step j's slice sits in LDS stage j % NWS; during step k the weights of step
  // k + 3 are loaded into registers and those of step k + 2 (loaded during step k - 1) are
  // stored at the step's end. Patches: stage g's patch sits in buffer g % 2; the next stage's
  // patch is loaded at step 0 of a stage and stored at step 4 (its buffer was last read in
  // step 7 of the previous stage). Fragments are read one half step (K = 16) ahead; one barrier
  // per step. (With KS = 2 the patch is stored at step 2 and first read in step 3.)
  Stage cur = stage_at(0, 0);
  Stage nxt = next_stage(cur);
  load_w(wreg[0], cur.col);
  store_w(wreg[0], 0);
  load_w(wreg[0], cur.col + p.Cip);
  store_w(wreg[0], 1);
  load_w(wreg[0], cur.col + 2 * p.Cip);  // step 2, stored at the end of step 0
  load_patch(preg, cur, true);
  store_patch(preg, 0);
  __syncthreads();
  read_a(wf[0], 0, 0);
  read_b(bf[0], 0, 0, 0);

  constexpr int NM = MB * NB;  // matrix ops per half step
  auto step = [&](auto PP, auto SS, int k, int g) {
    constexpr int P = decltype(PP)::value;  // stage parity: patch buffer
    constexpr int S = decltype(SS)::value;  // spatial tap
    constexpr int KP = (P * SPS + S) & 1;   // parity of k
    // half step 0 (step k + 3 lies in this stage or the next: SPS >= 4)
    load_w(wreg[KP ^ 1], S + 3 < SPS ? cur.col + (S + 3) * p.Cip : nxt.col + (S + 3 - SPS) * p.Cip);
    if constexpr (S == 0) load_patch(preg, nxt, g + 1 < ng);
    read_a(wf[1], S % NWS, 1);
    read_b(bf[1], P, S, 1);
    compute(wf[0], bf[0]);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x006, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // half step 1
    read_a(wf[0], (S + 1) % NWS, 0);
    if constexpr (S < SPS - 1) read_b(bf[0], P, S + 1, 0);
    else read_b(bf[0], P ^ 1, 0, 0);
    compute(wf[1], bf[1]);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x006, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    store_w(wreg[KP], (S + 2) % NWS);
    if constexpr (S == STORE_S) store_patch(preg, P ^ 1);
    __syncthreads();
  };
  auto stage = [&](auto PP, int g) {
    const int k = g * SPS;
    step(PP, std::integral_constant<int, 0>{}, k + 0, g);
    step(PP, std::integral_constant<int, 1>{}, k + 1, g);
    step(PP, std::integral_constant<int, 2>{}, k + 2, g);
    step(PP, std::integral_constant<int, 3>{}, k + 3, g);
    if constexpr (SPS == 9) {
      step(PP, std::integral_constant<int, 4>{}, k + 4, g);
      step(PP, std::integral_constant<int, 5>{}, k + 5, g);
      step(PP, std::integral_constant<int, 6>{}, k + 6, g);
      step(PP, std::integral_constant<int, 7>{}, k + 7, g);
      step(PP, std::integral_constant<int, 8>{}, k + 8, g);
    }
    cur = nxt;
    nxt = next_stage(nxt);
  };
  int g = 0;
  for (; g + 1 < ng; g += 2) {
    stage(std::integral_constant<int, 0>{}, g);
    stage(std::integral_constant<int, 1>{}, g + 1);
  }
  if (g < ng) stage(std::integral_constant<int, 0>{}, g);

  conv_epilogue<NB, MB, NORM>(p, acc, ph, pw, pv, tf, n0, pa, pb, half);
  run_copy_share(p.copy);
}

// LDS-DMA variant of the 3x3-tap halo kernel. Same tiles, K order, fragments and epilogue; the
// staging goes straight from memory into LDS with buffer loads that write LDS (each lane's 16
// bytes land at the instruction's LDS base + 16 * lane), so no registers, no LDS store
// instructions and no address arithmetic per piece. A weight row and a patch position are five
// 16-byte slots (32 channels and the pad); a lane that draws a pad slot, a slot past the rows, a
// position outside the frame or a channel past Ci reads out of range and writes zeros.
// Weights sit in six LDS slots, one per K step (step j in slot j % 6), and are fetched five
// steps ahead: slot (k + 5) % 6 last held step k - 1, which every wave finished before the
// barrier of step k - 1. The next stage's patch is fetched at step 0 of a stage into the other
// buffer (last read in the previous stage). Before the barrier of step k a wave waits until its
// own fetches up to step k - 3 have landed (a count of the fetches it issued since, fixed at
// compile time): that covers the weights of step k + 2 (read from step k + 1 on) and, from step
// 3, the next patch (read from step 8 on). Each slot and buffer is its own LDS array, so the
// compiler's own waits before LDS reads only cover fetches into the array being read.
// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 fields: vmcnt bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8; expcnt 7 and lgkmcnt 15 do not wait).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Workgroup barrier for the DMA kernels' LDS traffic. The builtin alone is an intrinsic that
// touches no memory as far as the compiler is concerned, so LDS loads and stores could be moved
// across it; the empty asm statements with a memory clobber on both sides pin every memory
// access to its side of the barrier. They emit no instruction and, unlike a workgroup fence,
// add no s_waitcnt (the fetches still in flight are covered by the hand-counted vmcnt waits).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until this wave's LDS operations (the fused tail's accumulations, which return nothing, so
// the compiler waits for none of them) are done: lgkmcnt 0 only.
__device__ __forceinline__ void lds_ops_done() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Waves per SIMD a DMA kernel is compiled for: two, or four for the one-row phase tiles (their
// light main loop leaves the SIMDs to the epilogue's vector work, which other waves then overlap).
template <int NB, int MB, int KS>
constexpr int dma_waves_per_simd() { return (KS == 2 && MB == 1 && NB <= 3) ? 4 : 2; }

template <int NB, int MB, int WAVES, int KS, bool NORM, bool DUAL = false, bool TAIL = false, bool SC = false>
__global__ __launch_bounds__(WAVES * 64, TAIL ? 1 : (dma_waves_per_simd<NB, MB, KS>() * 4 / WAVES)) void conv_halo_dma_kernel(
    const ConvProblem p) {
  static_assert(KS == 2 || KS == 3, "3x3 taps, or 2x2 phase taps");
  static_assert(!TAIL || (KS == 2 && NB == 3 && MB == 1 && WAVES == 8 && NORM && !DUAL), "the fused tail's tile");
  static_assert(!SC || (KS == 2 && NB == 6 && MB == 1 && WAVES == 8 && DUAL && !TAIL), "the shortcut product's tile");
  constexpr int SPS = KS * KS;
  // weight fetch distance D (steps ahead), slots NWS (> D, and k mod NWS a compile-time
  // function of the stage parity and the tap), barrier wait window WW = D - 2 steps (must not
  // exceed SPS - 2 so that the patch fetched at step 0 is in place for step SPS - 1)
  // (2x2 taps on 8-row tiles: D = 3 and 4 slots, and 3x3 taps on 4-wave 8-row tiles: D = 2 and 3
  // slots, so that two workgroups fit in one CU's LDS; 128-wide channel tiles: D = 2 and 3 slots
  // of 16 KB beside the 96 KB of patches)
  constexpr bool SMALL = (SPS == 4 && WAVES * MB == 8);
  constexpr bool SMALL3 = (SPS == 9 && (WAVES == 4 || NB == 4));
  constexpr int D = (SPS == 9) ? (SMALL3 ? 2 : 5) : (SMALL ? 3 : 4);
  constexpr int NWS = (SPS == 9) ? (SMALL3 ? 3 : 6) : (SMALL ? 4 : 8), WW = D - 2;
  static_assert(WW <= SPS - 2 && D < NWS && (2 * SPS) % NWS == 0, "fetch distance, slots and wait window");
  constexpr int BN = NB * 32;
  constexpr int TR = WAVES * MB;
  // patch: the tile with a 1-pixel halo; 2x2 phase taps need one side only (the side set by
  // the phase), so their patch starts at (h0 - 1 + a, w0 - 1 + b) and is one row and column smaller
  constexpr int PR = TR + (KS == 3 ? 2 : 1), PC = (KS == 3 ? 34 : 33);
  constexpr int PSLOTS = PR * PC * 5;                                // 16-byte slots of a patch
  constexpr int PIW = (PSLOTS + 64 * WAVES - 1) / (64 * WAVES);      // patch fetches per wave
  constexpr int WSLOTS = BN * 5;                                     // 16-byte slots of a weight step
  constexpr int WIW = (WSLOTS + 64 * WAVES - 1) / (64 * WAVES);      // weight fetches per wave
  constexpr int PBYTES = PIW * WAVES * 1024, WBYTES = WIW * WAVES * 1024;
  static_assert(2 * PBYTES + NWS * WBYTES <= 163840, "LDS");
  // Output staging at a tile's end (conv_epilogue_staged): the patch buffer of the tile's last
  // stage is idle (the other one holds the next tile's first patch, possibly still in flight).
  // NBP: the widest pass (96, 64 or 32 channels) whose per-wave areas all fit in it. (One known
  // LDS array, so the compiler's waits before the staging accesses do not cover the prefetch.)
  constexpr auto staging_fits = [](int nbp) constexpr { return PBYTES / (32 * (nbp * 64 + 16)) >= WAVES; };
  constexpr int NBP = (NB % 3 == 0 && staging_fits(3)) ? 3 : ((NB % 2 == 0 && staging_fits(2)) ? 2 : 1);
  static_assert(staging_fits(NBP), "staging areas");
  __shared__ __attribute__((aligned(16))) bf16_t lds_p0[PBYTES / 2];
  __shared__ __attribute__((aligned(16))) bf16_t lds_p1[PBYTES / 2];
  __shared__ __attribute__((aligned(16))) bf16_t lds_w0[WBYTES / 2];
  __shared__ __attribute__((aligned(16))) bf16_t lds_w1[WBYTES / 2];
  __shared__ __attribute__((aligned(16))) bf16_t lds_w2[WBYTES / 2];
  __shared__ __attribute__((aligned(16))) bf16_t lds_w3[WBYTES / 2];
  __shared__ __attribute__((aligned(16))) bf16_t lds_w4[WBYTES / 2];
  __shared__ __attribute__((aligned(16))) bf16_t lds_w5[WBYTES / 2];
  __shared__ __attribute__((aligned(16))) bf16_t lds_w6[NWS > 6 ? WBYTES / 2 : 8];
  __shared__ __attribute__((aligned(16))) bf16_t lds_w7[NWS > 6 ? WBYTES / 2 : 8];
  // The fused tail (TAIL): the head's weights as the first operand of the Z product (row m a
  // tap-colour of one temporal tap, the 96 channels in the activation operand's order, rows of
  // 104 elements: 16-byte reads of 32 rows are conflict free) and the frame's output accumulator
  // (the 18 x 66 output pixels around the block's 16 x 64 activated positions; per pixel and
  // colour a 16-byte group of the three temporal taps' sums and a pad).
  constexpr int TZR = 104, TCR = 2 * TR + 2, TCC = 66, TCP = 12;
  __shared__ __attribute__((aligned(16))) bf16_t lds_hz[TAIL ? 96 * TZR : 8];
  // The shortcut product's weight (SC): 96 rows of 192 channels, rows 196 elements apart (392
  // bytes: the 8-byte operand reads of 32 rows fall on distinct banks), loaded once per
  // workgroup; beside the 112 KB of the 192-wide phase tile it still fits the CU's LDS.
  constexpr int SCR = 196;
  __shared__ __attribute__((aligned(16))) bf16_t lds_sc[SC ? 96 * SCR : 4];
  __shared__ __attribute__((aligned(16))) float lds_tc[TAIL ? TCR * TCC * TCP : 4];
  auto wslot = [&](auto I) -> bf16_t* {
    constexpr int i = decltype(I)::value;
    static_assert(i >= 0 && i < NWS, "slot");
    if constexpr (i == 0) return lds_w0;
    else if constexpr (i == 1) return lds_w1;
    else if constexpr (i == 2) return lds_w2;
    else if constexpr (i == 3) return lds_w3;
    else if constexpr (i == 4) return lds_w4;
    else if constexpr (i == 5) return lds_w5;
    else if constexpr (i == 6) return lds_w6;
    else return lds_w7;
  };
  auto pbuf = [&](auto I) -> bf16_t* {
    if constexpr (decltype(I)::value == 0) return lds_p0;
    else return lds_p1;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // Walking several tiles per workgroup keeps the tile loop's state live through the epilogue,
  // which the fused-norm epilogue cannot afford without spilling at four waves per SIMD; those
  // kernels take one tile. The fused tail (one workgroup per CU, two waves per SIMD) walks the
  // frames and phases of its block.
  constexpr bool PERSIST = !NORM || TAIL;
  // Tiles. The x2 phase convs deal their four phases as the fastest index: the four tiles of a
  // position run side by side, share its input patch in L2 and write neighbouring outputs close
  // in time. Each XCD owns a contiguous range of tiles (workgroup b runs on XCD b % 8); within
  // it workgroup `local` takes tiles local, local + G8, local + 2 G8, ... (G8 workgroups per XCD,
  // gridDim.x a multiple of 8), so an XCD always works on a window of neighbouring tiles. With
  // more than one tile per workgroup, the first stage of the next tile (its patch and the
  // weights of its first D steps) is fetched during the last stage of the current one, and its
  // matrix work starts right after the epilogue, while that epilogue's stores drain.
  constexpr int NPH = (KS == 2) ? 4 : 1;
  const int numR = (p.H + TR - 1) / TR, numC = (p.W + 31) / 32;
  const int tpf = numR * numC;
  const int numN = (p.Npad + BN - 1) / BN;
  const int total = p.T * tpf * numN * NPH;
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3, G8 = gridDim.x >> 3;
  const int q8 = total >> 3, r8 = total & 7;
  const int xs = xcd * q8 + (xcd < r8 ? xcd : r8), xl = q8 + (xcd < r8 ? 1 : 0);
  // The fused tail: workgroup -> a block of TR input rows x 32 columns at input row
  // -1 + k (TR - 1), column -1 + m 31 (neighbouring blocks share a row or column: the head's
  // 3x3 stencil needs the activated positions around its output tile, the block's 2 TR x 64
  // positions less a one-pixel border), blocks dealt in contiguous ranges per XCD; its tiles are
  // (frame, phase) in order. Otherwise a strided walk over the XCD's tile range.
  int tb_h0 = 0, tb_w0 = 0;
  int it_first = local, it_step = G8, it_end = xl;
  if constexpr (TAIL) {
    const int nbr = (2 * p.H + 2 * TR - 2) / (2 * TR - 2), nbc = (2 * p.W + 62) / 62;
    const int nblk = nbr * nbc, per = (nblk + 7) >> 3;
    const int blk = xcd * per + local;
    if (blk >= nblk) return;  // (uniform)
    tb_h0 = -1 + (blk / nbc) * (TR - 1);
    tb_w0 = -1 + (blk - (blk / nbc) * nbc) * 31;
    it_first = 0;
    it_step = 1;
    it_end = 4 * p.T;
  } else if (local >= xl) {  // no tile for this workgroup (uniform)
    run_copy_share(p.copy);
    return;
  }
  struct Tile {
    int tf, h0, w0, n0, phase;
  };
  auto decode = [&](int it) -> Tile {
    if constexpr (TAIL) return {it >> 2, tb_h0, tb_w0, 0, it & 3};
    const int lin_p = xs + it;
    const int phase = lin_p % NPH, lin = lin_p / NPH;
    const int mt = lin / numN, nt = lin - (lin / numN) * numN;
    const int tf = p.time_tiles ? mt % p.T : mt / tpf;
    const int rem = p.time_tiles ? mt / p.T : mt - tf * tpf;
    const int rt = rem / numC;
    return {tf, rt * TR, (rem - rt * numC) * 32, nt * BN, phase};
  };
  const int dt0 = -2 * (p.kt >> 1);
  const int nchunks = p.Cip >> 5;
  const int ng = nchunks * p.kt;
  const int64_t frame_elems = (int64_t)p.H * p.W * p.Ci;
  const uint32_t frame_bytes = (uint32_t)(frame_elems * 2);
  const int64_t wrow = (int64_t)p.ntaps * p.Cip;
  // the tile's packed weight rows (phase, n0 ..): rows past Npad lie past the range and read 0
  auto weight_rsrc = [&](const Tile& t) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(p.wpk + ((int64_t)t.phase * p.Npad + t.n0) * wrow), (short)0,
                                             (int)((int64_t)(p.Npad - t.n0) * wrow * 2), 0x00020000);
  };

  // B operand of tap (0, 0): patch position (r + 1 + dh0, l32 + 1 + dw0) (tile independent)
  uint32_t boff[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    boff[mb] = (uint32_t)((((wave * MB + mb) * PC + l32) * PROW + half * 16) * 2);
  // This lane's patch slots: byte offset in a frame for chunk 0 (or frame_bytes: always zero)
  // and the slot's channel group (for the Ci tail of the last chunk).
  uint32_t pgo[PIW];
  int pch[PIW];
  // (recomputed from an opaque copy of the thread index at each tile: hoisting the
  // tile-independent part out of the tile loop would hold 2 * PIW more registers through it)
  auto patch_offsets = [&](const Tile& t) __attribute__((always_inline)) {
    const int pa = (KS == 2) ? (t.phase >> 1) : 0, pb = (KS == 2) ? (t.phase & 1) : 0;
    int ltid = tid;
    asm volatile("" : "+v"(ltid));
#pragma unroll
    for (int i = 0; i < PIW; ++i) {
      const int j = i * WAVES * 64 + ltid;
      const int pos = j / 5, part = j - (j / 5) * 5;
      const int pr = pos / PC, pc = pos - (pos / PC) * PC;
      const int hh = t.h0 - 1 + pa + pr, ww = t.w0 - 1 + pb + pc;
      const bool ok = (part < 4) & (pos < PR * PC) & (hh >= 0) & (hh < p.H) & (ww >= 0) & (ww < p.W);
      pgo[i] = ok ? (uint32_t)(((hh * p.W + ww) * p.Ci + part * 8) * 2) : frame_bytes;
      pch[i] = part * 8;
    }
  };
  // This lane's weight slots: byte offset of (row, 8-channel group) in the packed rows; pads and
  // slots past the tile's BN rows read past any tile's range (zero, no memory traffic).
  uint32_t wgo[WIW];
#pragma unroll
  for (int i = 0; i < WIW; ++i) {
    const int j = (i * WAVES + wave) * 64 + lane;
    const int row = j / 5, part = j - (j / 5) * 5;
    wgo[i] = (part < 4 && row < BN) ? (uint32_t)((row * wrow + part * 8) * 2) : 0x7ffffff0u;
  }

  typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
  typedef __attribute__((address_space(3))) void lds_void;
  u32x4 wf[2][NB];
  u32x4 bf[2][MB];

  // A stage of the K loop: 32-channel chunk, temporal tap i, weight column; nt: in the next tile
  struct Stage {
    int chunk, i, col, nt;
  };
  auto stage_at = [&](int chunk, int i, int nt) -> Stage { return {chunk, i, i * SPS * p.Cip + chunk * 32, nt}; };
  auto next_stage = [&](const Stage& c) -> Stage {
    if (c.chunk * p.kt + c.i + 1 >= ng) return stage_at(0, 0, 1);
    return (c.i + 1 == p.kt) ? stage_at(c.chunk + 1, 0, c.nt) : stage_at(c.chunk, c.i + 1, c.nt);
  };

  int it = it_first;                            // the current tile
  bool more = PERSIST && it + it_step < it_end;  // whether there is a next tile
  Tile tc = decode(it);
  Tile tn = more ? decode(it + it_step) : tc;
  __amdgpu_buffer_rsrc_t rs_cur = weight_rsrc(tc), rs_nxt = weight_rsrc(tn);

  // fetch a stage's patch (of the current or the next tile) into buffer BUF (live == false: zeros)
  auto fetch_patch = [&](auto BUF, const Stage& c, bool live) __attribute__((always_inline)) {
    const int sf = (c.nt ? tn.tf : tc.tf) + dt0 + c.i;
    const bool fok = live & (sf >= -p.Th);
    const bf16_t* fbase = (sf >= 0) ? p.x + (int64_t)sf * frame_elems
                                    : ((sf >= -p.Th) ? p.hist + (int64_t)(sf + p.Th) * frame_elems : p.x);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)fbase, (short)0, fok ? (int)frame_bytes : 0, 0x00020000);
    char* base = (char*)pbuf(BUF);
#pragma unroll
    for (int i = 0; i < PIW; ++i) {
      const uint32_t vo = (c.chunk * 32 + pch[i] < p.Ci) ? pgo[i] + c.chunk * 64 : frame_bytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(base + (i * WAVES + wave) * 1024), 16, (int)vo, 0, 0, 0);
    }
  };
  // fetch the weights of one K step (column col of the packed rows) into slot SLOT
  auto fetch_w = [&](auto SLOT, int col, __amdgpu_buffer_rsrc_t rs) {
    char* base = (char*)wslot(SLOT);
#pragma unroll
    for (int i = 0; i < WIW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(base + (i * WAVES + wave) * 1024), 16,
                                               (int)(wgo[i] + col * 2), 0, 0, 0);
  };
  auto read_a = [&](u32x4 (&dst)[NB], auto SLOT, int q) {
    const bf16_t* w = wslot(SLOT);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) dst[nb] = *(const u32x4*)(&w[(nb * 32 + l32) * LDS_ROW + half * 16 + q * 8]);
  };
  auto read_b = [&](u32x4 (&dst)[MB], auto BUF, int tap, int q) {
    const int j = tap / KS, k = tap - (tap / KS) * KS;
    const char* base = (const char*)pbuf(BUF);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) dst[mb] = *(const u32x4*)(base + boff[mb] + ((j * PC + k) * PROW + q * 8) * 2);
  };

  floatx16 acc[NB][MB];
  auto zero_acc = [&]() {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.0f;
  };
  auto compute = [&](const u32x4 (&w)[NB], const u32x4 (&a)[MB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w[nb]),
                                                              __builtin_bit_cast(bf16x8, a[mb]), acc[nb][mb], 0, 0, 0);
  };

  // The fused tail's output pixels of this thread: px = tid + 512 u of the block's
  // (2 TR - 2) x 62 output tile (video row 2 tb_h0 + 1 + px / 62, column 2 tb_w0 + 1 + px % 62),
  // with the partial sums of the next two output frames (their temporal tap 0 and 1 terms).
  constexpr int TOR = 2 * TR - 2, TOC = 62;
  float to0[2][3], to1[2][3];
  auto tail_pixel = [&](int u, int& Yo, int& Xo) -> bool {
    const int px = tid + WAVES * 64 * u;
    const int orow = px / TOC, ocol = px - (px / TOC) * TOC;
    Yo = 2 * tb_h0 + 1 + orow;
    Xo = 2 * tb_w0 + 1 + ocol;
    return (px < TOR * TOC) & (Yo >= 0) & (Yo < 2 * p.H) & (Xo >= 0) & (Xo < 2 * p.W);
  };
  if constexpr (TAIL) {
    // Z product operand: row m = 32 bz + r holds temporal tap bz of tap-colour (jk, o) where,
    // with ri = (r / 8) * 4 + r % 4 the accumulator register and hf = (r / 4) % 2 the lane half
    // that hold row r, (jk, o) = (ri, hf) for ri < 9 and (2 (ri - 9) + hf, 2) for 9 <= ri < 14
    // (every lane then adds whole registers per spatial tap); its 96 channels in the order the
    // activation operand holds them: K16 chunk q, half h2, element i8 is channel
    // (q / 2) * 32 + (2 (q % 2) + i8 / 4) * 8 + h2 * 4 + i8 % 4.
    for (int idx = tid; idx < 96 * 96; idx += WAVES * 64) {
      const int m = idx / 96, kk = idx - (idx / 96) * 96;
      const int bz = m >> 5, r = m & 31;
      const int ri = (r >> 3) * 4 + (r & 3), hf = (r >> 2) & 1;
      const int jk = ri < 9 ? ri : 2 * (ri - 9) + hf, o = ri < 9 ? hf : 2;
      const int q = kk >> 4, h2 = (kk >> 3) & 1, i8 = kk & 7;
      const int c = (q >> 1) * 32 + (2 * (q & 1) + (i8 >> 2)) * 8 + h2 * 4 + (i8 & 3);
      bf16_t v = 0;
      if (ri < 14 && jk < 9 && o < p.head_co && c < p.N) v = p.head_w[((int64_t)(jk * 4 + o) * 3 + bz) * p.Cip + c];
      lds_hz[m * TZR + kk] = v;
    }
    for (int idx = tid; idx < TCR * TCC * TCP; idx += WAVES * 64) lds_tc[idx] = 0.0f;
    const int64_t plane = (int64_t)(2 * p.H) * (2 * p.W);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int Yo, Xo;
      const bool own = tail_pixel(u, Yo, Xo) && p.carry_valid;
      const int64_t at = (int64_t)Yo * (2 * p.W) + Xo;
#pragma unroll
      for (int o = 0; o < 3; ++o) {
        to0[u][o] = own ? p.carry[o * plane + at] : 0.0f;
        to1[u][o] = own ? p.carry[(3 + o) * plane + at] : 0.0f;
      }
    }
  }

  // SC: this thread's 16-byte pieces of the shortcut weight (96 rows x 24 pieces), fetched
  // before the prologue's fetches and written to LDS after its full wait
  constexpr int SCN = SC ? (96 * 24 + WAVES * 64 - 1) / (WAVES * 64) : 1;
  uint4 scv[SCN];
  if constexpr (SC) {
#pragma unroll
    for (int i = 0; i < SCN; ++i) {
      const int j = i * WAVES * 64 + tid;
      scv[i] = j < 96 * 24 ? *(const uint4*)(p.sc_w + (int64_t)(j / 24) * p.sc_wrow + (j % 24) * 8)
                           : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  // prologue: the first tile's first stage (patch and steps 0 .. D - 1, all in stage 0)
  patch_offsets(tc);
  Stage cur = stage_at(0, 0, 0);
  Stage nxt = next_stage(cur);
  fetch_patch(I0{}, cur, true);
  fetch_w(I0{}, cur.col, rs_cur);
  fetch_w(I1{}, cur.col + p.Cip, rs_cur);
  if constexpr (D >= 3) fetch_w(I2{}, cur.col + 2 * p.Cip, rs_cur);
  if constexpr (D >= 4) fetch_w(I3{}, cur.col + 3 * p.Cip, rs_cur);
  if constexpr (D == 5) fetch_w(I4{}, cur.col + 4 * p.Cip, rs_cur);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  if constexpr (SC) {
#pragma unroll
    for (int i = 0; i < SCN; ++i) {
      const int j = i * WAVES * 64 + tid;
      if (j < 96 * 24) {
        uint2* d = (uint2*)(lds_sc + (j / 24) * SCR + (j % 24) * 8);
        d[0] = make_uint2(scv[i].x, scv[i].y);
        d[1] = make_uint2(scv[i].z, scv[i].w);
      }
    }
  }
  lds_barrier();
  read_a(wf[0], I0{}, 0);
  read_b(bf[0], I0{}, 0, 0);
  zero_acc();

  constexpr int NM = MB * NB;
  // The first stage of a tile that follows an epilogue in this workgroup (persistent tiles):
  // every fetch issued before that epilogue has landed (it starts with a full wait), so that
  // stage's first WW steps, whose waits would cover only such fetches, wait for nothing. (A
  // count there would also have to count the epilogue's stores, which the counter may retire
  // out of order with the fetches: LLVM's own waits treat mixed loads and stores that way.)
  bool fresh = false;
  auto step = [&](auto PP, auto SS) __attribute__((always_inline)) {
    constexpr int P = decltype(PP)::value;  // stage parity: patch buffer
    constexpr int S = decltype(SS)::value;  // spatial tap
    constexpr int K6 = (P * SPS + S) % NWS;  // k mod NWS (k = SPS * g + S)
    __builtin_amdgcn_sched_barrier(0);
    // step k + D lies in this stage or the next one (D < 2 * SPS - S), which may be the next
    // tile's first stage
    if constexpr (S + D < SPS) {
      fetch_w(std::integral_constant<int, (K6 + D) % NWS>{}, cur.col + (S + D) * p.Cip, rs_cur);
    } else {
      fetch_w(std::integral_constant<int, (K6 + D) % NWS>{}, nxt.col + (S + D - SPS) * p.Cip,
              nxt.nt ? rs_nxt : rs_cur);
    }
    if constexpr (S == 0) {
      if (PERSIST && nxt.nt) patch_offsets(tn);  // the current tile fetches no more patches
      fetch_patch(std::integral_constant<int, P ^ 1>{}, nxt, !nxt.nt || more);
    }
    __builtin_amdgcn_sched_barrier(0);
    read_a(wf[1], std::integral_constant<int, K6>{}, 1);
    read_b(bf[1], std::integral_constant<int, P>{}, S, 1);
    compute(wf[0], bf[0]);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x006, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    read_a(wf[0], std::integral_constant<int, (K6 + 1) % NWS>{}, 0);
    if constexpr (S < SPS - 1) read_b(bf[0], std::integral_constant<int, P>{}, S + 1, 0);
    else read_b(bf[0], std::integral_constant<int, P ^ 1>{}, 0, 0);
    compute(wf[1], bf[1]);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x006, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // own fetches of steps <= k - WW have landed: the ones issued in steps k - WW + 1 .. k may not
    constexpr int N = WW * WIW + (S < WW ? PIW : 0);
    static_assert(N < 64, "vmcnt range");
    if constexpr (PERSIST && S < WW) {
      if (!fresh) __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
    }
    lds_barrier();
  };
  auto stage = [&](auto PP) __attribute__((always_inline)) {
    step(PP, I0{});
    step(PP, I1{});
    step(PP, I2{});
    step(PP, I3{});
    if constexpr (SPS == 9) {
      step(PP, I4{});
      step(PP, std::integral_constant<int, 5>{});
      step(PP, std::integral_constant<int, 6>{});
      step(PP, std::integral_constant<int, 7>{});
      step(PP, std::integral_constant<int, 8>{});
    }
    fresh = false;
    cur = nxt;
    if (!nxt.nt) nxt = next_stage(nxt);  // (past a tile's last stage nxt is set at the switch)
  };
  // After each stage: at a tile's end (its last stage of parity PL) the epilogue, then the
  // switch to the next tile, whose first stage (parity PL ^ 1) is already fetched. Returns
  // whether the workgroup is done.
  if constexpr (!PERSIST) {
    // One tile: its stages, then the epilogue with both patch buffers (and two weight slots if
    // needed) as staging areas once every fetch has landed.
    int g = 0;
    for (; g + 1 < ng; g += 2) {
      stage(I0{});
      stage(I1{});
    }
    if (g < ng) stage(I0{});
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    const int pa = (KS == 2) ? (tc.phase >> 1) : 0, pb = (KS == 2) ? (tc.phase & 1) : 0;
    int ph[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) ph[mb] = tc.h0 + wave * MB + mb;
    if (p.staged) {
      lds_barrier();
      constexpr auto fits1 = [](int nbp) constexpr {
        const int sb = 32 * (nbp * 64 + 16);
        return 2 * (PBYTES / sb) + 2 * (WBYTES / sb) >= WAVES;
      };
      constexpr int NBP1 = (NB % 3 == 0 && fits1(3)) ? 3 : ((NB % 2 == 0 && fits1(2)) ? 2 : 1);
      constexpr int SB = StagedShape<NBP1>::BYTES, PCAP = PBYTES / SB, WCAP = WBYTES / SB > 0 ? WBYTES / SB : 1;
      static_assert(fits1(NBP1), "staging areas");
      char* st;
      if (wave < PCAP) st = (char*)lds_p0 + wave * SB;
      else if (wave < 2 * PCAP) st = (char*)lds_p1 + (wave - PCAP) * SB;
      else {
        const int r = wave - 2 * PCAP;
        st = ((r / WCAP == 0) ? (char*)wslot(I0{}) : (char*)wslot(I1{})) + (r % WCAP) * SB;
      }
      conv_epilogue_staged<NB, MB, NORM, NBP1, DUAL, SC>(p, acc, ph, tc.w0, tc.tf, tc.n0, pa, pb, lane, st,
                                                         lds_sc);
    } else if constexpr (!DUAL) {  // (the launcher stages every dual-store launch)
      int pw[MB];
      bool pv[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        pw[mb] = tc.w0 + l32;
        pv[mb] = (ph[mb] < p.H) & (pw[mb] < p.W);
      }
      conv_epilogue<NB, MB, NORM>(p, acc, ph, pw, pv, tc.tf, tc.n0, pa, pb, half);
    }
    run_copy_share(p.copy);
    return;
  }
  // The fused tail's epilogue of one phase tile: norm_out + SiLU of the accumulators (the plain
  // fused-norm arithmetic) into bf16 operands, positions outside the frame zero (the head's
  // padding); Z = head weights x activations (81 tap-colour rows of the three temporal taps:
  // three 32-row blocks, K = 96); then every Z value is added into the frame's output
  // accumulator at the pixel its spatial tap (j, k) serves, (Y - j + 1, X - k + 1), by plain
  // reads, adds and writes of 16-byte groups (colour o: the three temporal taps). No two of them
  // meet in one batch of reads and writes: within a wave, spatial taps k = 0 and 2 of
  // neighbouring lanes meet at one pixel and run in two batches, in order (a wave's LDS
  // operations complete in order); rows j = 0 and 2 of neighbouring waves meet and are separated
  // by a barrier (j = 1 meets neither); the phases of a frame are separated by the main loop's
  // barriers. So every sum is taken in one fixed order.
  auto tail_epilogue = [&](const Tile& t) __attribute__((always_inline)) {
    const int pa = t.phase >> 1, pb = t.phase & 1;
    const int hh = t.h0 + wave, ww = t.w0 + l32;
    const bool inside = (hh >= 0) & (hh < p.H) & (ww >= 0) & (ww < p.W);
    const float* bias = opaque(p.bias);
    const float* gamma = opaque(p.norm_gamma);
    float ss = 0.0f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = nb * 32 + g * 8;
        if (c >= p.N) continue;  // (wave-uniform)
        const float4 b4 = bias ? *(const float4*)(bias + c + half * 4) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = acc[nb][0][g * 4 + e] + bv[e];
          acc[nb][0][g * 4 + e] = v;
          ss = fmaf(v, v, ss);
        }
      }
    ss += __shfl_xor(ss, 32, 64);
    const float inv_n = 1.0f / (float)p.N;
    const float rs = rsqrtf(ss * inv_n + p.norm_eps);
    u32x4 xo[6];
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      const int nb = q >> 1;
      float v[8];
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int g = (q & 1) * 2 + gg;
        const int c = nb * 32 + g * 8;
        float4 gm = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (c < p.N) gm = *(const float4*)(gamma + c + half * 4);
        const float gv[4] = {gm.x, gm.y, gm.z, gm.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float a = acc[nb][0][g * 4 + e] * rs * gv[e];
          if (p.norm_silu) a = silu_f32(a);
          v[gg * 4 + e] = (inside && c < p.N) ? a : 0.0f;
        }
      }
      xo[q][0] = pack_bf16x2(v[0], v[1]);
      xo[q][1] = pack_bf16x2(v[2], v[3]);
      xo[q][2] = pack_bf16x2(v[4], v[5]);
      xo[q][3] = pack_bf16x2(v[6], v[7]);
    }
    floatx16 z[3];
#pragma unroll
    for (int bz = 0; bz < 3; ++bz)
#pragma unroll
      for (int r = 0; r < 16; ++r) z[bz][r] = 0.0f;
#pragma unroll
    for (int q = 0; q < 6; ++q)
#pragma unroll
      for (int bz = 0; bz < 3; ++bz) {
        const u32x4 a = *(const u32x4*)(&lds_hz[(bz * 32 + l32) * TZR + q * 16 + half * 8]);
        z[bz] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, xo[q]),
                                                        z[bz], 0, 0, 0);
      }
    // accumulator index of pixel (Y + 1, X + 1) of this lane's position (Y, X) = (2 hh + pa,
    // 2 ww + pb), the block's pixel rows and columns counted from (2 h0 - 1, 2 w0 - 1); a lane adds
    // colour `half` of every spatial tap, and colour 2 of the taps jk with jk % 2 == half
    const int rb = 2 * wave + pa + 2, cb = 2 * l32 + pb + 2;
    auto batch = [&](auto J0, auto NJ, auto K0, auto NK) __attribute__((always_inline)) {
      constexpr int j0 = decltype(J0)::value, nj = decltype(NJ)::value;
      constexpr int k0 = decltype(K0)::value, nk = decltype(NK)::value;
      float4 r[nj][nk], r2[nj][nk];
#pragma unroll
      for (int a = 0; a < nj; ++a)
#pragma unroll
        for (int b = 0; b < nk; ++b) {
          const int jk = (j0 + a) * 3 + k0 + b;
          const float* t = lds_tc + ((rb - j0 - a) * TCC + (cb - k0 - b)) * TCP;
          r[a][b] = *(const float4*)(t + half * 4);
          if (half == (jk & 1)) r2[a][b] = *(const float4*)(t + 8);
        }
#pragma unroll
      for (int a = 0; a < nj; ++a)
#pragma unroll
        for (int b = 0; b < nk; ++b) {
          const int jk = (j0 + a) * 3 + k0 + b;
          float* t = lds_tc + ((rb - j0 - a) * TCC + (cb - k0 - b)) * TCP;
          r[a][b].x += z[0][jk];
          r[a][b].y += z[1][jk];
          r[a][b].z += z[2][jk];
          *(float4*)(t + half * 4) = r[a][b];
          if (half == (jk & 1)) {
            r2[a][b].x += z[0][9 + (jk >> 1)];
            r2[a][b].y += z[1][9 + (jk >> 1)];
            r2[a][b].z += z[2][9 + (jk >> 1)];
            *(float4*)(t + 8) = r2[a][b];
          }
        }
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    // (the empty asm statements keep the compiler from moving a batch's reads above the previous
    // batch's writes: the address another lane wrote is one this thread never wrote)
    batch(C0{}, C2{}, C0{}, C2{});  // rows j = 0, 1, columns k = 0, 1
    asm volatile("" ::: "memory");
    batch(C0{}, C2{}, C2{}, C1{});  // rows j = 0, 1, column k = 2
    lds_ops_done();
    lds_barrier();
    batch(C2{}, C1{}, C0{}, C2{});  // row j = 2, columns k = 0, 1
    asm volatile("" ::: "memory");
    batch(C2{}, C1{}, C2{}, C1{});  // row j = 2, column k = 2
  };
  // After a frame's last phase: output frame tf is complete (its tap 2 term is this frame's),
  // + bias, one bf16 rounding into the video; the partial sums move on by a frame
  // (sum order of an output frame f: ((tap 0 of f - 2) + tap 1 of f - 1) + tap 2 of f); the
  // accumulator is cleared for the next frame.
  auto tail_finish = [&](int tf) __attribute__((always_inline)) {
    lds_ops_done();
    lds_barrier();  // every wave's sums of the frame are in
    const float* hb = opaque(p.head_b);
    const int64_t plane = (int64_t)(2 * p.H) * (2 * p.W);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int Yo, Xo;
      const bool own = tail_pixel(u, Yo, Xo);
      const int px = tid + WAVES * 64 * u;
      if (px < TOR * TOC) {
        const int orow = px / TOC, ocol = px - (px / TOC) * TOC;
        const float* src = lds_tc + ((orow + 2) * TCC + ocol + 2) * TCP;
#pragma unroll
        for (int o = 0; o < 3; ++o) {
          const float4 cv = *(const float4*)(src + 4 * o);  // temporal taps 0, 1, 2 of colour o
          const float f = to0[u][o] + cv.z;
          if (own && o < p.head_co)
            p.video[((int64_t)o * p.video_frames + p.video_fbase + tf) * plane + (int64_t)Yo * (2 * p.W) + Xo] =
                (bf16_t)f32_to_bf16(f + (hb ? hb[o] : 0.0f));
          to0[u][o] = to1[u][o] + cv.y;
          to1[u][o] = cv.x;
        }
      }
    }
    lds_barrier();  // every read of the frame's sums is done
    for (int idx = tid; idx < TCR * TCC * TCP / 4; idx += WAVES * 64)
      *(float4*)(lds_tc + 4 * idx) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    lds_ops_done();
  };
  int g = 0;  // stage within the tile
  auto after_stage = [&](auto PL) __attribute__((always_inline)) -> bool {
    constexpr int L = decltype(PL)::value;
    if (++g < ng) return false;
    g = 0;
    // every fetch this wave issued (the next tile's first patch and weights among them) lands
    // before the epilogue's loads and stores go out (see `fresh`); the epilogue's first bias read
    // waited for them anyway
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    const int pa = (KS == 2) ? (tc.phase >> 1) : 0, pb = (KS == 2) ? (tc.phase & 1) : 0;
    int ph[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) ph[mb] = tc.h0 + wave * MB + mb;
    if constexpr (TAIL) {
      (void)ph;
      tail_epilogue(tc);
      if (tc.phase == 3) tail_finish(tc.tf);
    } else if (p.staged) {
      // Staging areas: the finished stage's patch buffer and, since nothing is in flight now, the
      // weight slot of the next tile's step D (fetched only at that tile's first step, after the
      // barrier that closes this epilogue): the widest pass whose per-wave areas fit in both.
      constexpr auto fits_pw = [](int nbp) constexpr {
        const int sb = 32 * (nbp * 64 + 16);
        return PBYTES / sb + WBYTES / sb >= WAVES;
      };
      constexpr int NBQ = (NB % 3 == 0 && fits_pw(3)) ? 3 : ((NB % 2 == 0 && fits_pw(2)) ? 2 : 1);
      constexpr int SBQ = StagedShape<NBQ>::BYTES, PCAPQ = PBYTES / SBQ;
      constexpr int FREE = (((L ^ 1) * SPS) + D) % NWS;
      char* st = wave < PCAPQ ? (char*)pbuf(PL) + wave * SBQ
                              : (char*)wslot(std::integral_constant<int, FREE>{}) + (wave - PCAPQ) * SBQ;
      conv_epilogue_staged<NB, MB, NORM, NBQ>(p, acc, ph, tc.w0, tc.tf, tc.n0, pa, pb, lane, st);
    } else {
      int pw[MB];
      bool pv[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        pw[mb] = tc.w0 + l32;
        pv[mb] = (ph[mb] < p.H) & (pw[mb] < p.W);
      }
      conv_epilogue<NB, MB, NORM>(p, acc, ph, pw, pv, tc.tf, tc.n0, pa, pb, half);
    }
    if (!more) return true;
    it += it_step;
    more = PERSIST && it + it_step < it_end;
    tc = tn;
    rs_cur = rs_nxt;
    if (more) {
      tn = decode(it + it_step);
      rs_nxt = weight_rsrc(tn);
    }
    cur.nt = 0;
    nxt = next_stage(cur);
    fresh = true;
    zero_acc();
    // every wave is done with the staging areas before the next tile's fetches reuse them
    lds_barrier();
    read_a(wf[0], std::integral_constant<int, ((L ^ 1) * SPS) % NWS>{}, 0);
    read_b(bf[0], std::integral_constant<int, L ^ 1>{}, 0, 0);
    return false;
  };
  for (;;) {
    stage(I0{});
    if (after_stage(I0{})) break;
    stage(I1{});
    if (after_stage(I1{})) break;
  }
  // fetches past the end (into slots and buffers nobody reads) land before the workgroup exits
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  if constexpr (TAIL) {
    // the partial sums of the two frames after the pass, for the next one
    const int64_t plane = (int64_t)(2 * p.H) * (2 * p.W);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int Yo, Xo;
      if (!tail_pixel(u, Yo, Xo)) continue;
      const int64_t at = (int64_t)Yo * (2 * p.W) + Xo;
#pragma unroll
      for (int o = 0; o < 3; ++o) {
        p.carry[o * plane + at] = to0[u][o];
        p.carry[(3 + o) * plane + at] = to1[u][o];
      }
    }
  }
  run_copy_share(p.copy);
}

// LDS-DMA GEMM for the convolutions without spatial taps (1x1x1 convs and the (3,1,1) time conv):
// the K loop of the linear kernel (32-channel chunk outermost, temporal taps inside, the same
// operand layout per lane, so the same sums bit for bit), with both operands staged through LDS
// by buffer loads that write LDS. A workgroup owns BM = WM * 64 positions of one frame x BN =
// WN * NB * 32 channels; its waves form a WM x WN grid, each 64 positions x NB * 32 channels
// (two position blocks and NB channel blocks: every fragment read from LDS feeds two or NB
// matrix ops). A K step stages BM activation rows and BN weight rows of 32 channels (64 bytes
// each) in one of four LDS stages; a row's four 16-byte pieces are stored XOR-swizzled by bits
// 2-3 of the row, so the fragment reads of 16 consecutive rows fall on distinct banks without a
// pad. Step k fetches step k + 3 into the stage that step k - 1 finished; before the barrier
// that ends step k each wave waits for its own fetches of step k + 2 (the fragments of its first
// half are read during step k + 1). Two tile shapes: 4 waves (2 x 2, 128 x 192 or 128 x 128,
// 80 or 64 KB of LDS), two workgroups per CU so that one's epilogue overlaps the other's matrix
// work; and 8 waves (4 x 2, 256 x 256, 128 KB), one per CU, whose LDS traffic per matrix op is
// a fifth lower (each staged row feeds more of them), for grids that fill the chip. The epilogue
// is the staged one, a position row of 32 at a time.
template <int NB, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64, (WM * WN == 4) ? 2 : 1) void conv_gemm_dma_kernel(const ConvProblem p) {
  constexpr int WAVES = WM * WN, MB = 2;
  static_assert((WM == 2 && WN == 2) || (WM == 4 && WN == 2 && NB == 4), "the 4- and 8-wave tiles");
  constexpr int BM = WM * MB * 32;          // positions per tile
  constexpr int BN = WN * NB * 32;          // channels per tile
  constexpr int ALOADS = BM * 4 / 64;      // 1 KB loads of a step's activation rows
  constexpr int BLOADS = BN * 4 / 64;      // and of its weight rows
  static_assert(ALOADS % WAVES == 0 && BLOADS % WAVES == 0, "loads per wave");
  constexpr int AIW = ALOADS / WAVES, BIW = BLOADS / WAVES, LPW = AIW + BIW;
  constexpr int SBYTES = (ALOADS + BLOADS) * 1024;
  static_assert(4 * SBYTES <= (WAVES == 4 ? 81920 : 163840), "LDS (4 waves: two workgroups per CU)");
  __shared__ __attribute__((aligned(16))) bf16_t lds_s0[SBYTES / 2];
  __shared__ __attribute__((aligned(16))) bf16_t lds_s1[SBYTES / 2];
  __shared__ __attribute__((aligned(16))) bf16_t lds_s2[SBYTES / 2];
  __shared__ __attribute__((aligned(16))) bf16_t lds_s3[SBYTES / 2];
  auto sbuf = [&](auto I) -> bf16_t* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return lds_s0;
    else if constexpr (i == 1) return lds_s1;
    else if constexpr (i == 2) return lds_s2;
    else return lds_s3;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int wm = wave % WM, wn = wave / WM;

  // Tile: frame tf, positions m0 .. m0 + BM - 1 of it, channels n0 .. n0 + BN - 1. Each XCD
  // takes a contiguous range of tiles, channel tiles fastest (they share the activation rows in
  // L2), then the frames of one position range (the temporal taps of neighbouring frames meet
  // in L2).
  const int HW = p.H * p.W;
  const int tpf = (HW + BM - 1) / BM;
  const int numN = (p.Npad + BN - 1) / BN;
  const int total = p.T * tpf * numN;
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int q8 = total >> 3, r8 = total & 7;
  const int lin = xcd * q8 + (xcd < r8 ? xcd : r8) + local;
  const int mt = lin / numN, nt = lin - (lin / numN) * numN;
  const int tf = mt % p.T, m0 = (mt / p.T) * BM, n0 = nt * BN;

  const int dt0 = -2 * (p.kt >> 1);
  const int nchunks = p.Cip >> 5;
  const int nk = p.kt * nchunks;
  const int64_t frame_elems = (int64_t)HW * p.Ci;
  const uint32_t frame_bytes = (uint32_t)(frame_elems * 2);
  const int64_t wrow = (int64_t)p.ntaps * p.Cip;
  const bf16_t* wbase = p.wpk + (int64_t)n0 * wrow;
  const __amdgpu_buffer_rsrc_t rs_w =
      __builtin_amdgcn_make_buffer_rsrc((void*)wbase, (short)0, (int)((int64_t)(p.Npad - n0) * wrow * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_dead = __builtin_amdgcn_make_buffer_rsrc((void*)wbase, (short)0, 0, 0x00020000);

  // This lane's pieces: load L (of its wave) covers rows 16 L .. 16 L + 15 of the stage, lane l
  // the row's LDS piece l % 4, which holds its 8-channel group l % 4 ^ (l / 16) % 4.
  const int part = (lane & 3) ^ ((lane >> 4) & 3);
  uint32_t aoff[AIW], boff[BIW];
#pragma unroll
  for (int i = 0; i < AIW; ++i) {
    const int m = m0 + (i * WAVES + wave) * 16 + (lane >> 2);
    aoff[i] = m < HW ? (uint32_t)((m * p.Ci + part * 8) * 2) : frame_bytes;
  }
#pragma unroll
  for (int i = 0; i < BIW; ++i) {
    const int row = (i * WAVES + wave) * 16 + (lane >> 2);
    boff[i] = (uint32_t)((row * wrow + part * 8) * 2);
  }
  // Fragment reads: row base + l32 (base a multiple of 32), 16-byte group half * 2 + q.
  uint32_t fo[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) fo[q] = (uint32_t)(l32 * 64 + (((half * 2 + q) ^ ((l32 >> 2) & 3)) * 16));

  typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
  typedef __attribute__((address_space(3))) void lds_void;

  struct Cur {
    int step, chunk, ti;
  };
  auto advance = [&](Cur& c) {
    const bool wrap = c.ti + 1 == p.kt;
    c.ti = wrap ? 0 : c.ti + 1;
    c.chunk += wrap ? 1 : 0;
    c.step += 1;
  };
  // fetch K step c into stage SS (steps past the last one read nothing and write zeros)
  auto fetch = [&](auto SS, const Cur& c) __attribute__((always_inline)) {
    char* base = (char*)sbuf(SS);
    const bool live = c.step < nk;
    const int sf = tf + dt0 + c.ti;
    const bool fok = live & (sf >= -p.Th);
    const bf16_t* fb = (sf >= 0) ? p.x + (int64_t)sf * frame_elems
                                 : ((sf >= -p.Th) ? p.hist + (int64_t)(sf + p.Th) * frame_elems : p.x);
    const __amdgpu_buffer_rsrc_t rs_a =
        __builtin_amdgcn_make_buffer_rsrc((void*)fb, (short)0, fok ? (int)frame_bytes : 0, 0x00020000);
    const bool cok = c.chunk * 32 + part * 8 < p.Ci;
#pragma unroll
    for (int i = 0; i < AIW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, (lds_void*)(base + (i * WAVES + wave) * 1024), 16,
                                               (int)(cok ? aoff[i] + c.chunk * 64 : frame_bytes), 0, 0, 0);
    const int col = c.ti * p.Cip + c.chunk * 32;
    const __amdgpu_buffer_rsrc_t rs_b = live ? rs_w : rs_dead;
#pragma unroll
    for (int i = 0; i < BIW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, (lds_void*)(base + (ALOADS + i * WAVES + wave) * 1024), 16,
                                               (int)(boff[i] + col * 2), 0, 0, 0);
  };

  u32x4 wf[2][NB];
  u32x4 af[2][MB];
  auto read_frags = [&](u32x4 (&w)[NB], u32x4 (&a)[MB], auto SS, int q) __attribute__((always_inline)) {
    const char* base = (const char*)sbuf(SS);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      w[nb] = *(const u32x4*)(base + (BM + (wn * NB + nb) * 32) * 64 + fo[q]);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) a[mb] = *(const u32x4*)(base + ((wm * MB + mb) * 32) * 64 + fo[q]);
  };

  floatx16 acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.0f;
  auto compute = [&](const u32x4 (&w)[NB], const u32x4 (&a)[MB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w[nb]),
                                                              __builtin_bit_cast(bf16x8, a[mb]), acc[nb][mb], 0, 0, 0);
  };

  // prologue: steps 0, 1, 2 into stages 0, 1, 2; steps 0 and 1 landed before the first reads
  Cur cf = {0, 0, 0};
  fetch(I0{}, cf);
  advance(cf);
  fetch(I1{}, cf);
  advance(cf);
  fetch(I2{}, cf);
  advance(cf);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPW));
  lds_barrier();
  read_frags(wf[0], af[0], I0{}, 0);

  constexpr int NM = MB * NB;
  auto step = [&](auto SS) __attribute__((always_inline)) {
    constexpr int S = decltype(SS)::value;  // k % 4
    __builtin_amdgcn_sched_barrier(0);
    fetch(std::integral_constant<int, (S + 3) & 3>{}, cf);  // step k + 3, into the stage of step k - 1
    advance(cf);
    __builtin_amdgcn_sched_barrier(0);
    read_frags(wf[1], af[1], SS, 1);
    compute(wf[0], af[0]);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x006, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    read_frags(wf[0], af[0], std::integral_constant<int, (S + 1) & 3>{}, 0);  // step k + 1's first half
    compute(wf[1], af[1]);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x006, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // own fetches of step k + 2 have landed (only step k + 3's may still be in flight)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPW));
    lds_barrier();
  };
  int k = 0;
  for (; k + 4 <= nk; k += 4) {
    step(I0{});
    step(I1{});
    step(I2{});
    step(I3{});
  }
  const int rem = nk - k;
  if (rem > 0) step(I0{});
  if (rem > 1) step(I1{});
  if (rem > 2) step(I2{});

  // the fetches past the last step land before the stages become staging areas
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();
  constexpr int NBP = (NB % 3 == 0) ? 3 : ((NB % 2 == 0) ? 2 : 1);
  constexpr int SB = StagedShape<NBP>::BYTES;
  constexpr int CAP = SBYTES / SB;  // staging areas per stage
  static_assert(2 * CAP >= WAVES, "staging areas");
  char* st = wave < CAP ? (char*)lds_s0 + wave * SB : (char*)lds_s1 + (wave - CAP) * SB;
  // the frame as one row of H*W positions: a wave's 32 positions are consecutive in the output
  ConvProblem q = p;
  q.H = 1;
  q.W = HW;
  q.Ho = 1;
  q.Wo = HW;
  const int row0[1] = {0};
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    floatx16 a1[NB][1];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) a1[nb][0] = acc[nb][mb];
    conv_epilogue_staged<NB, 1, false, NBP>(q, a1, row0, m0 + (wm * MB + mb) * 32, tf, n0 + wn * NB * 32, 0, 0,
                                            lane, st);
  }
  run_copy_share(p.copy);
}

// DMA conv kernels without a fused norm run persistent workgroups (one per resident slot,
// several tiles each).
constexpr bool kPersistentDmaTiles = true;
constexpr int kNumCUs = 256;

struct ConfigEntry {
  const char* name;
  int nb, mb, waves;
  int halo;  // conv_halo_kernel's KS (WAVES*MB rows x 32 columns per tile), or 0
  int time_tiles;  // halo tile order (ConvProblem::time_tiles)
  int phase_in_x;  // the x2 phases are part of the linear block index (grid z = 1)
  int staged;      // the kernel has the LDS-staged epilogue (used when ConvProblem allows it)
  int wgs_per_cu;  // workgroups resident per CU (a DMA kernel then walks several tiles each)
  int gemm;        // conv_gemm_dma_kernel's WM (waves along the positions; waves / WM along the
                   // channels, each mb x nb blocks), one tile per workgroup; or 0
  void (*kernel)(const ConvProblem);       // plain epilogue (bias, residual, fp32 planes)
  void (*kernel_norm)(const ConvProblem);  // fused RMS norm (+ SiLU) epilogue
  void (*kernel_dual)(const ConvProblem);  // fused norm + the pre-norm value stored too (or null)
};

#define WVD_CONV_CONFIG(NB, MB, W) \
  { "conv_mfma_n" #NB "_m" #MB "_w" #W, NB, MB, W, 0, 0, 0, 0, 0, 0, conv_mfma_kernel<NB, MB, W, false>, \
    conv_mfma_kernel<NB, MB, W, true>, nullptr }
// 3x3-tap halo convs order tiles time-fastest (measured 2-8% faster than frame-major on every
// 3x3x3 layer: fewer input re-reads past L2); the phase convs have no temporal taps.
#define WVD_HALO_CONFIG(NB, MB, W) \
  { "conv_halo_n" #NB "_m" #MB "_w" #W, NB, MB, W, 3, 1, 0, 0, 0, 0, conv_halo_kernel<NB, MB, W, 3, false>, \
    conv_halo_kernel<NB, MB, W, 3, true>, nullptr }
#define WVD_HALO_DMA_CONFIG(NB, MB, W) \
  { "conv_halo_dma_n" #NB "_m" #MB "_w" #W, NB, MB, W, 3, 1, 0, 1, dma_waves_per_simd<NB, MB, 3>() * 4 / W, \
    0, conv_halo_dma_kernel<NB, MB, W, 3, false>, \
    conv_halo_dma_kernel<NB, MB, W, 3, true>, nullptr }
// (the one-tile widths a residual block's conv2 takes at 96 and 192 channels: also the dual store)
#define WVD_HALO_DMA_DUAL_CONFIG(NB, MB, W) \
  { "conv_halo_dma_n" #NB "_m" #MB "_w" #W, NB, MB, W, 3, 1, 0, 1, dma_waves_per_simd<NB, MB, 3>() * 4 / W, \
    0, conv_halo_dma_kernel<NB, MB, W, 3, false>, \
    conv_halo_dma_kernel<NB, MB, W, 3, true>, conv_halo_dma_kernel<NB, MB, W, 3, true, true> }
// (no fused-norm instantiation: the norm needs every channel in one tile, and the 96- and 192-wide
// tiles cover those widths)
#define WVD_HALO_DMA_PLAIN_CONFIG(NB, MB, W) \
  { "conv_halo_dma_n" #NB "_m" #MB "_w" #W, NB, MB, W, 3, 1, 0, 1, dma_waves_per_simd<NB, MB, 3>() * 4 / W, \
    0, conv_halo_dma_kernel<NB, MB, W, 3, false>, nullptr, nullptr }
#define WVD_PHASE_HALO_DMA_CONFIG(NB, MB, W) \
  { "conv_phase_halo_dma_n" #NB "_m" #MB "_w" #W, NB, MB, W, 2, 0, 1, 1, dma_waves_per_simd<NB, MB, 2>() * 4 / W, \
    0, conv_halo_dma_kernel<NB, MB, W, 2, false>, \
    conv_halo_dma_kernel<NB, MB, W, 2, true>, nullptr }
// (192 channels in one tile, for a fused norm of that width with the pre-norm value stored too:
// the x2 upsample that feeds a 192-channel residual block)
#define WVD_PHASE_HALO_DMA_DUAL_CONFIG(NB, MB, W) \
  { "conv_phase_halo_dma_n" #NB "_m" #MB "_w" #W, NB, MB, W, 2, 0, 1, 1, dma_waves_per_simd<NB, MB, 2>() * 4 / W, \
    0, conv_halo_dma_kernel<NB, MB, W, 2, false>, \
    conv_halo_dma_kernel<NB, MB, W, 2, true>, conv_halo_dma_kernel<NB, MB, W, 2, true, true> }
// The fused tail: the x2 phase conv with norm_out + SiLU and the output head in one kernel (only
// for problems with head_w set, never chosen or forced for others).
#define WVD_TAIL_CONFIG(NB, MB, W) \
  { "conv_tail_phase_head_n" #NB "_m" #MB "_w" #W, NB, MB, W, 2, 0, 1, 1, 0, \
    0, conv_halo_dma_kernel<NB, MB, W, 2, true, false, true>, conv_halo_dma_kernel<NB, MB, W, 2, true, false, true>, \
    nullptr }
// The 192-wide x2 phase tile with the dual store whose pre-norm value is replaced by its 1x1
// product (ConvProblem::y_sc; only for problems with y_sc set, never chosen or forced for others).
#define WVD_PHASE_SC_CONFIG(NB, MB, W) \
  { "conv_phase_halo_dma_sc_n" #NB "_m" #MB "_w" #W, NB, MB, W, 2, 0, 1, 1, dma_waves_per_simd<NB, MB, 2>() * 4 / W, \
    0, conv_halo_dma_kernel<NB, MB, W, 2, true, true, false, true>, conv_halo_dma_kernel<NB, MB, W, 2, true, true, false, true>, \
    conv_halo_dma_kernel<NB, MB, W, 2, true, true, false, true> }
#define WVD_GEMM_DMA_CONFIG(NB, WM, WN) \
  { "conv_gemm_dma_n" #NB "_m2_w" #WM "x" #WN, NB, 2, WM * WN, 0, 0, 0, 1, 0, WM, conv_gemm_dma_kernel<NB, WM, WN>, \
    nullptr, nullptr }
#define WVD_PHASE_HALO_CONFIG(NB, MB, W) \
  { "conv_phase_halo_n" #NB "_m" #MB "_w" #W, NB, MB, W, 2, 0, 0, 0, 0, 0, conv_halo_kernel<NB, MB, W, 2, false>, \
    conv_halo_kernel<NB, MB, W, 2, true>, nullptr }

// Two waves per SIMD (8-wave workgroups, or two 4-wave workgroups per CU) measured faster than
// bigger per-wave tiles at one wave per SIMD: the second wave issues matrix work while the first
// waits on memory.
// Configuration ids: indices into kConfigs (also the timing and force-config indices).
enum ConfigId {
  LIN_N6_W8,     // 192 x 256, 2 waves/SIMD
  LIN_N6_W4,     // 192 x 128, 2 workgroups/CU
  LIN_N3_W8,     // 96 x 256, 2 waves/SIMD
  LIN_N3_W4,     // 96 x 128: small grids
  LIN_N1_M4_W4,  // 32 x 512: a few output channels
  LIN_N3_M2_W8,  // 96 x 512, 2 waves/SIMD: long reductions (3x3x3 taps)
  HALO_N6_W8,    // 192 x (8 rows x 32 columns)
  HALO_N3_W8,    // 96 x (16 rows x 32 columns)
  HALO_N3_W4,    // 96 x (8 rows x 32 columns), two workgroups per CU
  PHASE_N6_W8,   // x2 upsampling phases: 192 x (8 rows x 32 columns)
  PHASE_N3_W8,   // x2 upsampling phases: 96 x (16 rows x 32 columns)
  HALO_DMA_N3_W8,  // HALO_N3_W8 with LDS-DMA staging
  HALO_DMA_N6_W8,  // HALO_N6_W8 with LDS-DMA staging
  PHASE_DMA_N3_W8,  // PHASE_N3_W8 with LDS-DMA staging
  PHASE_DMA_N3_W4,  // x2 upsampling phases: 96 x (8 rows x 32 columns), two workgroups per CU
  PHASE_DMA_N3_M1_W8,  // the same tile, one row per wave: two 8-wave workgroups per CU
  HALO_DMA_N2_W8,  // 64 x (16 rows x 32 columns): small grids
  HALO_DMA_N1_W8,  // 32 x (16 rows x 32 columns): a few output channels (a 12-channel head)
  LIN_N4_W8,       // 128 x 256, 2 waves/SIMD: channel counts that are multiples of 128, not of 96
  HALO_DMA_N3_W4,  // 96 x (8 rows x 32 columns) on 4 waves in 80 KB: two workgroups per CU
  HALO_DMA_N4_W8,  // 128 x (16 rows x 32 columns): channel counts that are multiples of 128, not of 96
  PHASE_DMA_N6_M1_W8,  // x2 upsampling phases: 192 x (8 rows x 32 columns), one row per wave, 112 KB
  TAIL_N3_M1_W8,       // the fused tail: PHASE_DMA_N3_M1_W8's tiles, all phases and frames of a block
  PHASE_DMA_SC_N6_M1_W8,  // PHASE_DMA_N6_M1_W8's dual store with the shortcut product (y_sc)
  GEMM_N3_W4,      // 1x1 and (3,1,1) convs: 192 x 128 GEMM tiles, both operands LDS-DMA staged
  GEMM_N2_W4,      // the same, 128 x 128: channel counts that are multiples of 128, not of 192
  GEMM_N4_W8,      // 256 x 256 on 8 waves, one workgroup per CU: grids that fill the chip
  NUM_CONFIGS
};
const ConfigEntry kConfigs[] = {
    WVD_CONV_CONFIG(6, 1, 8),       WVD_CONV_CONFIG(6, 1, 4),       WVD_CONV_CONFIG(3, 1, 8),
    WVD_CONV_CONFIG(3, 1, 4),       WVD_CONV_CONFIG(1, 4, 4),       WVD_CONV_CONFIG(3, 2, 8),
    WVD_HALO_CONFIG(6, 1, 8),       WVD_HALO_CONFIG(3, 2, 8),       WVD_HALO_CONFIG(3, 2, 4),
    WVD_PHASE_HALO_CONFIG(6, 1, 8), WVD_PHASE_HALO_CONFIG(3, 2, 8), WVD_HALO_DMA_DUAL_CONFIG(3, 2, 8),
    WVD_HALO_DMA_DUAL_CONFIG(6, 1, 8), WVD_PHASE_HALO_DMA_CONFIG(3, 2, 8), WVD_PHASE_HALO_DMA_CONFIG(3, 2, 4),
    WVD_PHASE_HALO_DMA_CONFIG(3, 1, 8), WVD_HALO_DMA_CONFIG(2, 2, 8),    WVD_HALO_DMA_CONFIG(1, 2, 8),
    WVD_CONV_CONFIG(4, 1, 8),           WVD_HALO_DMA_CONFIG(3, 2, 4),    WVD_HALO_DMA_PLAIN_CONFIG(4, 2, 8),
    WVD_PHASE_HALO_DMA_DUAL_CONFIG(6, 1, 8), WVD_TAIL_CONFIG(3, 1, 8), WVD_PHASE_SC_CONFIG(6, 1, 8),
    WVD_GEMM_DMA_CONFIG(3, 2, 2),       WVD_GEMM_DMA_CONFIG(2, 2, 2),    WVD_GEMM_DMA_CONFIG(4, 4, 2),
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);
static_assert(kNumConfigs == NUM_CONFIGS, "one table entry per ConfigId");
constexpr int kMaxFusedNormN = 192;  // the widest channel tile
constexpr int round_up_int(int v, int m) { return (v + m - 1) / m * m; }

// Workgroups of a problem: per frame ceil(H*W / BM) position tiles (halo kernels: ceil(H / rows)
// x ceil(W / 32)), times the channel tiles.
int64_t blocks_for(const ConfigEntry& c, int64_t T, int64_t H, int64_t W, int Npad) {
  if (c.gemm) {
    const int64_t bn = (int64_t)c.nb * 32 * (c.waves / c.gemm), bm = (int64_t)c.mb * 32 * c.gemm;
    return T * ((H * W + bm - 1) / bm) * ((Npad + bn - 1) / bn);
  }
  const int64_t bn = (int64_t)c.nb * 32;
  const int64_t nt = (Npad + bn - 1) / bn;
  if (c.halo) {
    const int64_t tr = (int64_t)c.waves * c.mb;
    return T * ((H + tr - 1) / tr) * ((W + 31) / 32) * nt;
  }
  const int64_t bm = (int64_t)c.waves * c.mb * 32;
  return T * ((H * W + bm - 1) / bm) * nt;
}

// The GEMM kernel's problems: no spatial taps or phases, the plain output mapping (time-interleaved
// frames allowed), no fused norm, second output or fused tail, and the staged epilogue's
// conditions (bf16 output, N and nsplit multiples of 8, y and the residual 16-byte aligned).
bool gemm_fits(const ConvProblem& p) {
  const bool plain_map = p.phases == 1 && p.hmul == 1 && p.wmul == 1 && p.Ho == p.H && p.Wo == p.W;
  return plain_map && p.kh == 1 && p.kw == 1 && p.ntaps == p.kt && !p.norm_gamma && !p.y_pre && !p.y_sc &&
         !p.head_w && !p.y_f32 && p.Ci % 8 == 0 && p.N % 8 == 0 && p.nsplit % 8 == 0 &&
         ((uintptr_t)p.y & 15) == 0 && ((uintptr_t)p.res & 15) == 0;
}

// Convolutions with 3x3 spatial taps take the LDS-DMA halo kernel with 96 x (16 x 32) tiles
// (measured the fastest on every 3x3x3 layer of the decoder, 384-channel ones included: two
// position blocks per wave halve the weight fragment reads per matrix op; DMA staging 5-12 %
// faster than register staging), or its 192-wide variant when a fused norm needs more channels
// in one tile; 64-wide tiles on grids too small for the chip, 128-wide ones for channel counts
// that 96 does not divide, 8-row tiles on frames whose height a 16-row tile covers badly.
// Otherwise: the largest linear tile whose grid still gives every CU a workgroup per phase; a
// 96-wide channel tile takes two position blocks per wave on long reductions, one on short ones.
int choose_config(const ConvProblem& p, bool one_n_tile) {
  const int64_t cus = 256;
  const int64_t T = p.T, H = p.H, W = p.W;
  const int Npad = p.Npad, phases = p.phases;
  // (a dual store of at most 32 channels takes the 96-wide tile below, which has that epilogue)
  if (Npad <= 32 && phases == 1 && p.kh == 3 && p.kw == 3 && !p.y_pre) return HALO_DMA_N1_W8;
  if (Npad <= 32 && !(phases == 1 && p.kh == 3 && p.kw == 3)) return LIN_N1_M4_W4;
  if (phases == 1 && p.kh == 3 && p.kw == 3) {
    if (one_n_tile) return Npad > 96 ? HALO_DMA_N6_W8 : HALO_DMA_N3_W8;
    // a grid of 96-wide tiles that leaves CUs idle (the 4-frame 44x78 level: 144 tiles) takes
    // 64-wide ones if they still run in one round: two thirds of the tile time
    const int64_t b3 = blocks_for(kConfigs[HALO_DMA_N3_W8], T, H, W, Npad);
    const int64_t b2 = blocks_for(kConfigs[HALO_DMA_N2_W8], T, H, W, Npad);
    if (Npad % 64 == 0 && b3 < cus && b2 <= cus) return HALO_DMA_N2_W8;
    // channel counts that are multiples of 128 but not of 96 (1024, 512, 256) leave the last
    // 96-wide tile part empty; 128-wide tiles have none (and reuse each patch read over more
    // channels) when their rounds of tiles over the chip, each a third longer, take no longer:
    // measured 5-9 % faster at 1024, 512 and 256 channels on the 88x156 to 352x624 levels
    if (Npad % 128 == 0 && Npad % 96 != 0) {
      const int64_t b4 = blocks_for(kConfigs[HALO_DMA_N4_W8], T, H, W, Npad);
      if ((b4 + cus - 1) / cus * 4 <= (b3 + cus - 1) / cus * 3) return HALO_DMA_N4_W8;
    }
    // frames whose height leaves a 16-row tile mostly empty (the 88-row level: 96 rows tiled)
    // take the 8-row tiles, two workgroups per CU, about 5 % slower on whole tiles
    const int64_t r16 = (H + 15) / 16 * 16, r8 = (H + 7) / 8 * 8;
    return (r16 * 100 > r8 * 107) ? HALO_DMA_N3_W4 : HALO_DMA_N3_W8;
  }
  // The phase convs (K = 4 taps x C) have short reductions and heavy epilogues, so they run 8-row
  // DMA halo tiles with 80 KB of LDS, two workgroups per CU, whose epilogues overlap other waves'
  // matrix work: one row per wave (four waves per SIMD) measured fastest at 96 and 192 channels
  // (5-9 % over two rows per wave on 4 waves), two rows per wave at 384 (8 %).
  if (phases == 4 && p.kh == 2 && p.kw == 2 && (Npad <= 96 || (!one_n_tile && Npad <= 192)))
    return PHASE_DMA_N3_M1_W8;
  // a fused norm over 97-192 channels: all of them in one 192-wide phase tile
  if (phases == 4 && p.kh == 2 && p.kw == 2 && one_n_tile && Npad <= 192) return PHASE_DMA_N6_M1_W8;
  if (phases == 4 && p.kh == 2 && p.kw == 2 && !one_n_tile) return PHASE_DMA_N3_W4;
  // Convolutions without spatial taps (1x1x1, the (3,1,1) time conv) of at least 128 output
  // channels: the GEMM tiles. The 8-wave 256 x 256 tiles where their grid gives every CU a
  // workgroup and their width pads no more than the 4-wave ones (measured 15-36 % faster on the
  // decodes' big time convs and shortcuts, as fast on the 88x156 level); else 4-wave tiles, 192
  // wide unless 128-wide ones pad less
  if (Npad >= 128 && gemm_fits(p)) {
    const int p256 = (Npad + 255) / 256 * 256, p192 = (Npad + 191) / 192 * 192, p128 = (Npad + 127) / 128 * 128;
    if (p256 <= std::min(p192, p128) && blocks_for(kConfigs[GEMM_N4_W8], T, H, W, Npad) >= cus) return GEMM_N4_W8;
    return (p192 <= p128) ? GEMM_N3_W4 : GEMM_N2_W4;
  }
  const auto fills = [&](int id) { return blocks_for(kConfigs[id], T, H, W, Npad) * phases >= cus; };
  const int n96 = (p.ntaps >= 9 && fills(LIN_N3_M2_W8)) ? LIN_N3_M2_W8 : LIN_N3_W8;
  if (one_n_tile) {  // a fused norm needs every channel of a position in one workgroup
    if (Npad <= 96) return fills(LIN_N3_W8) ? n96 : LIN_N3_W4;
    return fills(LIN_N6_W8) ? LIN_N6_W8 : LIN_N6_W4;
  }
  // (256, 512, 1024 channels: 96- and 192-wide tiles would leave a third of a tile empty)
  if (Npad % 192 != 0 && Npad % 128 == 0 && fills(LIN_N4_W8)) return LIN_N4_W8;
  if (Npad % 192 == 0) {
    if (fills(LIN_N6_W8)) return LIN_N6_W8;
    if (fills(LIN_N6_W4)) return LIN_N6_W4;
    return LIN_N3_W4;
  }
  if (Npad % 96 == 0 && fills(LIN_N3_W8)) return n96;
  return LIN_N3_W4;
}

}  // namespace

bool conv_can_fuse_norm_width(int N) { return round_up_int(N, 32) <= kMaxFusedNormN && N % 8 == 0; }

bool conv_can_fuse_norm(int N, const float* bias, const float* gamma) {
  const auto a16 = [](const void* q) { return ((uintptr_t)q & 15u) == 0; };
  return conv_can_fuse_norm_width(N) && a16(bias) && a16(gamma) && gamma;
}

const char* conv_config_name(int id) { return (id >= 0 && id < kNumConfigs) ? kConfigs[id].name : "?"; }
int conv_config_count() { return kNumConfigs; }

// Whether configuration id can run p: halo tiles need 3x3 spatial taps without phases, a fused
// norm needs one channel tile.
bool conv_config_fits(const ConvProblem& p, int id) {
  if (id < 0 || id >= kNumConfigs) return false;
  if ((id == TAIL_N3_M1_W8) != (p.head_w != nullptr)) return false;
  if ((id == PHASE_DMA_SC_N6_M1_W8) != (p.y_sc != nullptr)) return false;
  const ConfigEntry& c = kConfigs[id];
  if (c.halo == 3 && !(p.phases == 1 && p.kh == 3 && p.kw == 3)) return false;
  if (c.halo == 2 && !(p.phases == 4 && p.kh == 2 && p.kw == 2)) return false;
  if (c.gemm && !gemm_fits(p)) return false;
  if (p.norm_gamma && (c.nb * 32 < p.Npad || !c.kernel_norm)) return false;
  if (p.y_pre && (!p.norm_gamma || !c.kernel_dual)) return false;
  return true;
}

bool tail_kernel_supported(int N, int Cip, int co) { return N > 64 && N <= 96 && N % 8 == 0 && Cip == 96 && co >= 1 && co <= 3; }

hipError_t launch_conv_mfma(const ConvProblem& p, hipStream_t s, int* config_id, int force_config,
                            int max_workgroups) {
  const int64_t HW = (int64_t)p.H * p.W;
  if (p.T == 0 || HW == 0) return hipSuccess;
  // one frame is addressed with 32-bit byte offsets
  if (HW * p.Ci * 2 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  // and one phase's packed weight rows (the DMA and GEMM tiles' weight buffer ranges)
  if ((int64_t)p.Npad * p.ntaps * p.Cip * 2 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if (p.head_w) {
    // the fused tail: an x2 phase conv of N -> N channels with norm_out + SiLU, no history,
    // residual or second output, a head of at most 3 colours; one workgroup per block
    if (force_config >= 0 && force_config != TAIL_N3_M1_W8) return hipErrorNotSupported;
    if (!tail_kernel_supported(p.N, p.Cip, p.head_co) || p.Ci != p.N || p.Npad != 96 || p.phases != 4 ||
        p.kh != 2 || p.kw != 2 || p.ntaps != 4 || !conv_can_fuse_norm(p.N, p.bias, p.norm_gamma) || p.res ||
        p.y_pre || p.hist || p.Th != 0 || !p.video || !p.carry || p.video_fbase < 0 ||
        p.video_fbase + (int64_t)p.T > p.video_frames)
      return hipErrorInvalidValue;
    const int64_t nbr = (2 * (int64_t)p.H + 14) / 14, nbc = (2 * (int64_t)p.W + 62) / 62;
    const int64_t gx = (nbr * nbc + 7) / 8 * 8;
    if (gx > 0x7fffffff || 4 * (int64_t)p.T > 0x7fffffff) return hipErrorInvalidValue;
    if (config_id) *config_id = TAIL_N3_M1_W8;
    ConvProblem q = p;
    q.time_tiles = 0;
    q.staged = 0;
    hipLaunchKernelGGL(kConfigs[TAIL_N3_M1_W8].kernel_norm, dim3((unsigned)gx), dim3(512), 0, s, q);
    return hipGetLastError();
  }
  // (a fused norm takes a residual only with the dual store, which adds it before the statistics)
  if (p.norm_gamma && (!conv_can_fuse_norm(p.N, p.bias, p.norm_gamma) || (p.res && !p.y_pre) || p.y_f32 ||
                       p.nsplit != p.N))
    return hipErrorInvalidValue;
  if (p.y_sc) {
    // the shortcut product in the dual store's place: the 192-wide x2 phase tile with a fused
    // norm, 96 shortcut outputs of all 192 channels, no pre-norm store or residual (the fused norm
    // keeps all channels in one frame: nsplit == N, checked below)
    if (!p.norm_gamma || p.y_pre || p.res || p.phases != 4 || p.kh != 2 || p.kw != 2 || p.N != 192 ||
        p.Npad != 192 || p.sc_co != 96 || !p.sc_w || p.sc_wrow < 192 || p.sc_wrow % 8 ||
        ((uintptr_t)p.sc_w & 15) || ((uintptr_t)p.sc_b & 15) || ((uintptr_t)p.y_sc & 15))
      return hipErrorInvalidValue;
  }
  int id = p.y_sc ? PHASE_DMA_SC_N6_M1_W8 : choose_config(p, p.norm_gamma != nullptr);
  if (force_config >= 0) {
    if (!conv_config_fits(p, force_config)) return hipErrorNotSupported;
    id = force_config;
  }
  const ConfigEntry& c = kConfigs[id];
  if (p.norm_gamma && !c.kernel_norm) return hipErrorNotSupported;
  if (p.y_pre && (!p.norm_gamma || !c.kernel_dual)) return hipErrorNotSupported;
  const int64_t blocks = blocks_for(c, p.T, p.H, p.W, p.Npad);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (config_id) *config_id = id;
  ConvProblem q = p;
  q.time_tiles = c.time_tiles;
  // the staged epilogue: the DMA kernels, and the linear kernel's one-block waves on the plain
  // output mapping (consecutive positions of a frame consecutive in the output)
  const bool plain_map = p.phases == 1 && p.hmul == 1 && p.wmul == 1 && p.Ho == p.H && p.Wo == p.W;
  const bool lin_staged = c.halo == 0 && c.mb == 1 && plain_map && !p.norm_gamma;
  q.staged = (c.staged || lin_staged) && !p.y_f32 && p.N % 8 == 0 && p.nsplit % 8 == 0 &&
             ((uintptr_t)p.y & 15) == 0 && ((uintptr_t)p.res & 15) == 0 && ((uintptr_t)p.y_pre & 15) == 0;
  if ((p.y_pre || p.y_sc) && !q.staged) return hipErrorNotSupported;  // the dual store exists staged only
  if (c.gemm && !q.staged) return hipErrorNotSupported;                // (gemm_fits implies staged)
  int64_t gx = c.phase_in_x ? blocks * p.phases : blocks;
  if (c.wgs_per_cu) {
    // DMA kernels: a multiple of 8 workgroups (XCD ranges); with persistent tiles no more than
    // fit on the chip at once, each walking its share of the tiles
    gx = (gx + 7) / 8 * 8;
    if (kPersistentDmaTiles && !p.norm_gamma) {
      gx = std::min<int64_t>(gx, (int64_t)kNumCUs * c.wgs_per_cu);
      if (max_workgroups > 0) gx = std::min<int64_t>(gx, std::max(8, max_workgroups / 8 * 8));
    }
  }
  if (gx > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((p.y_pre || p.y_sc) ? c.kernel_dual : (p.norm_gamma ? c.kernel_norm : c.kernel),
                     dim3((unsigned)gx, 1, c.phase_in_x ? 1 : p.phases),
                     dim3(c.waves * 64), 0, s, q);
  return hipGetLastError();
}

}  // namespace wvd
