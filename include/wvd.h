/*
 * wvd.h - C ABI of the MI355X (gfx950) causal-conv video decoder library (libwvd.so).
 *
 * What it computes is the decoder of the FastVideo compare page "[perf] PAN2 sampling: Wan2.2
 * VAE decode kernel, split decode, fused DiT kernels" (its reference decoder's docstring: the
 * part list, "The first latent frame yields one frame", "Causal caches", "Precision"), in a
 * synthetic topology: conv_in -> residual blocks -> up stages (residual blocks, a time conv on
 * temporal stages, a spatial x2 conv) -> RMS norm + SiLU -> conv_out. Each entry point below
 * names the part of that page it implements.
 *
 * Conventions shared by every entry point
 *  - Pure C: plain pointers and sizes. Device pointers are HIP device memory the CALLER owns
 *    (tensors, packed weights, cache storage, workspaces); the library allocates no device
 *    memory and keeps only small host structs (the cache handle).
 *  - Every call is asynchronous on the given hipStream_t (0 = the null stream). A call returns
 *    after enqueueing; results are ready when the stream reaches that point.
 *  - All argument validation happens before anything is enqueued: on an error nothing is
 *    launched, a wvd_status other than WVD_OK is returned and wvd_last_error() describes it.
 *    A launch failure reported by the HIP runtime is returned as WVD_ERR_HIP; a fault inside a
 *    kernel surfaces at the caller's next synchronisation.
 *  - Activations on bf16 paths are dense NTHWC ("channels last": [N][T][H][W][C], C innermost),
 *    batch N = 1. Sizes in wvd_tensor are the logical [N, C, T, H, W] sizes whatever the layout.
 *  - bf16 paths take bf16 operands, accumulate in fp32 and round each op's result to bf16 once
 *    (round to nearest even). The fp32 path computes in fp32.
 *  - Device pointers must be 16-byte aligned (WVD_ERR_ALIGN otherwise).
 *  - No function is safe to call concurrently on the same cache handle or workspace.
 */
#ifndef WVD_H
#define WVD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* wvd_stream; /* the same type as hipStream_t */

typedef enum {
  WVD_OK = 0,
  WVD_ERR_ARG = 1,         /* a null or out-of-range argument */
  WVD_ERR_SHAPE = 2,       /* tensor sizes do not fit together */
  WVD_ERR_DTYPE = 3,       /* wrong element type */
  WVD_ERR_LAYOUT = 4,      /* wrong memory layout */
  WVD_ERR_ALIGN = 5,       /* a device pointer is not 16-byte aligned */
  WVD_ERR_STATE = 6,       /* a cache handle used out of order, or for another decoder */
  WVD_ERR_WORKSPACE = 7,   /* the workspace is too small */
  WVD_ERR_UNSUPPORTED = 8, /* a shape or option this build does not implement */
  WVD_ERR_HIP = 9          /* the HIP runtime reported an error */
} wvd_status;

typedef enum { WVD_F32 = 0, WVD_BF16 = 1 } wvd_dtype;
typedef enum { WVD_NCTHW = 0, WVD_NTHWC = 1 } wvd_layout;

/* A dense 5-D tensor in device memory. n, c, t, h, w are the logical sizes. */
typedef struct {
  void* data;
  int32_t dtype;  /* wvd_dtype */
  int32_t layout; /* wvd_layout */
  int64_t n, c, t, h, w;
} wvd_tensor;

/* Message of the last failed call on this thread (valid until the next wvd_* call on it). */
const char* wvd_last_error(void);
/* ABI version; bumped on every incompatible change of this header. */
int wvd_abi_version(void);
#define WVD_ABI_VERSION 2

/* ============================================================================================
 * Layout conversion (boundary marshalling): NCTHW <-> NTHWC, fp32 <-> bf16 (round to nearest
 * even). x and y have the same logical sizes and must not overlap.
 * ========================================================================================== */
wvd_status wvd_convert(const wvd_tensor* x, wvd_tensor* y, wvd_stream stream);

/* ============================================================================================
 * Weight packing for the bf16 convolution kernels.
 *
 * WVD_PACK_CONV: raw [Co][Ci][kt][kh][kw] -> one phase, kt*kh*kw taps (causal conv part of the
 *   page: cross-correlation, tap i of kt meets frame t - (kt-1) + i).
 * WVD_PACK_PHASE2X: raw [Co][Ci][3][3] (a 2-D 3x3 conv applied after nearest x2 upsampling, the
 *   page's upsample2d part) -> four 2x2 "phase" kernels at the low resolution, one per output
 *   parity (a, b): each phase tap is the fp32 sum of the 3x3 taps that read the same low-res
 *   pixel, rounded once to bf16 (the kernel README's upsampler design: nearest x2 + 3x3 equals
 *   four 2x2 phase convolutions).
 * The raw weight is fp32 or bf16, dense, in device memory. `packed` is device memory of at least
 * wvd_conv_packed_bytes(...) bytes; its layout is private to the library (bf16, rows of output
 * channels padded to 32, taps, input channels padded to 32).
 * ========================================================================================== */
typedef enum { WVD_PACK_CONV = 0, WVD_PACK_PHASE2X = 1 } wvd_pack_mode;
size_t wvd_conv_packed_bytes(int co, int ci, int kt, int kh, int kw, int mode);
wvd_status wvd_conv_pack(const void* w_raw, int w_dtype, int co, int ci, int kt, int kh, int kw, int mode,
                         void* packed, wvd_stream stream);

/* ============================================================================================
 * wvd_causal_conv3d - one causal 3-D convolution (the page's causal conv part).
 *
 *   y[o,t,h,w] = bias[o] + sum_{c,i,j,k} W[o,c,i,j,k] * xt[c, t+i, h+j-kh/2, w+k-kw/2]
 *
 * with zero padding of kh/2, kw/2 in space and, in time, P = 2*(kt/2) frames in front of x: the
 * `hist` frames (oldest first) after P - hist.t zero frames. Stride 1, odd kernel sizes.
 *
 * bf16 path: x, hist, y bf16 NTHWC; `w` is packed (WVD_PACK_CONV) bf16; Ci % 8 == 0; fp32
 *   accumulation (implicit GEMM on the matrix cores). `residual` (nullable, bf16 NTHWC, the
 *   shape of y) is added before the single rounding of y.
 * fp32 path: x, hist, y fp32 in either layout (all the same layout); `w` is the RAW fp32 weight
 *   [Co][Ci][kt][kh][kw] (not packed); `residual` must be null.
 * bias: nullable fp32 [Co] in device memory.
 * hist: nullable, hist.t <= P, same c, h, w as x.
 * hist_out: nullable; when set, receives the history this conv leaves for the next chunk (the
 *   page's cached_conv rule: the last min(T, 2) input frames, or the old last history frame
 *   followed by x when x has one frame). Its t must be that frame count.
 * Aliasing: y may share no byte with x or hist, and hist_out none with x, hist or y (the
 *   workgroups read neighbouring rows and frames that others write); an overlap returns
 *   WVD_ERR_ARG before anything is launched.
 * x may have zero frames (so may the inputs of wvd_rmsnorm_silu, wvd_resblock and wvd_upsample;
 *   wvd_decode_chunk rejects an empty chunk): nothing is computed, y is empty, and the history
 *   passes through unchanged into hist_out.
 * ========================================================================================== */
wvd_status wvd_causal_conv3d(const wvd_tensor* x, const void* w, int co, int kt, int kh, int kw,
                             const float* bias, const wvd_tensor* hist, const wvd_tensor* residual, wvd_tensor* y,
                             wvd_tensor* hist_out, wvd_stream stream);

/* ============================================================================================
 * wvd_causal_conv3d_winograd - the causal 3x3x3 convolution of wvd_causal_conv3d (bf16 path,
 * same y, bias, hist and residual rules) computed with Winograd F(2x2, 3x3) in space and the
 * causal 3-tap time convolution kept as is, as the page's decoder runs its up blocks'
 * convolutions ("How the decoder got here", "The design"; there F(4x4, 3x3)). Each 2x2 output
 * tile takes the 4x4 input tile around it (zero outside the frame); its 16 transformed
 * components U = B^T d B (rounded to bf16) are multiplied with the transformed weights
 * V = G g G^T (bf16) on the matrix cores, summed over channels and time taps in fp32 (16 products
 * stored as fp32), and A^T M A + bias (+ residual) is rounded once into y. A layer-level
 * prototype (the decoder keeps the direct kernel): about 2.25x fewer products, three extra
 * memory-bound passes.
 * x, hist, residual, y: bf16 NTHWC; Ci % 8 == 0, co % 4 == 0; hist.t <= 2; y may share no byte
 * with x or hist. bias: nullable fp32 [co], 16-byte aligned. w_packed: from wvd_winograd_pack
 * (the raw weight [co][ci][3][3][3], fp32 or bf16), wvd_winograd_packed_bytes(co, ci) bytes,
 * 16-byte aligned. ws: wvd_winograd_workspace_bytes(ci, co, T, hist.t, H, W) bytes of device
 * memory (16 transformed input planes and 16 fp32 product planes), 16-byte aligned.
 * ========================================================================================== */
size_t wvd_winograd_packed_bytes(int co, int ci);
wvd_status wvd_winograd_pack(const void* w_raw, int w_dtype, int co, int ci, void* packed, wvd_stream stream);
size_t wvd_winograd_workspace_bytes(int ci, int co, int t, int th, int h, int w);
wvd_status wvd_causal_conv3d_winograd(const wvd_tensor* x, const void* w_packed, int co, const float* bias,
                                      const wvd_tensor* hist, const wvd_tensor* residual, wvd_tensor* y, void* ws,
                                      size_t ws_bytes, wvd_stream stream);

/* Channel RMS norm + SiLU (the page's RMS norm part, in the x * gamma / sqrt(mean_c x^2 + eps)
 * form; the SiLU of its residual block part): bf16 NTHWC in and out, fp32 statistics, one
 * rounding. gamma: fp32 [C] device memory. x and y may be the same tensor. */
wvd_status wvd_rmsnorm_silu(const wvd_tensor* x, const float* gamma, float eps, int apply_silu, wvd_tensor* y,
                            wvd_stream stream);

/* ============================================================================================
 * wvd_resblock - residual block (the page's residual block part):
 *   y = conv2(SiLU(norm2(conv1(SiLU(norm1(x)))))) + shortcut(x)
 * with 3x3x3 causal convs; the shortcut is x (cin == cout) or a 1x1x1 conv (cin != cout).
 * x: bf16 NTHWC [1, cin, T, H, W]; y: bf16 NTHWC [1, cout, T, H, W] (may not alias x).
 * hist1 / hist2: nullable activated histories (the conv inputs of the frames before x) for conv1
 * and conv2: bf16 NTHWC with c = cin / cout and t <= 2. hist1_out / hist2_out: nullable; receive
 * the histories for the next chunk (same rule as wvd_causal_conv3d; t = min(T,2) or hist.t + 1
 * for T == 1, capped at 2). The workspace must hold wvd_resblock_workspace_bytes(...) bytes.
 * ========================================================================================== */
typedef struct {
  int cin, cout;
  const float* gamma1;    /* [cin]  */
  const void* conv1;      /* packed WVD_PACK_CONV [cout, cin, 3,3,3] */
  const float* bias1;     /* [cout], nullable */
  const float* gamma2;    /* [cout] */
  const void* conv2;      /* packed [cout, cout, 3,3,3] */
  const float* bias2;     /* [cout], nullable */
  const void* shortcut;   /* packed [cout, cin, 1,1,1]; required iff cin != cout */
  const float* shortcut_bias; /* [cout], nullable */
} wvd_resblock_weights;

size_t wvd_resblock_workspace_bytes(int cin, int cout, int t, int h, int w);
wvd_status wvd_resblock(const wvd_tensor* x, const wvd_resblock_weights* wts, float eps, const wvd_tensor* hist1,
                        const wvd_tensor* hist2, wvd_tensor* y, wvd_tensor* hist1_out, wvd_tensor* hist2_out,
                        void* ws, size_t ws_bytes, wvd_stream stream);

/* wvd_resblock_noalloc - wvd_resblock without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). Same arguments, layouts, validation and results as wvd_resblock (it runs
 * the same kernels); the workspace is a scratch array built into the library, one per GPU,
 * wvd_resblock_noalloc_max_bytes() (32 MiB) long, kept until the process ends.
 * It calls no hipMalloc / hipFree and no allocating library routine (leave the per-launch
 * timing of wvd_timing_enable off: it creates HIP events).
 * Limit: inputs whose workspace, wvd_resblock_workspace_bytes(cin, cout, t, h, w), exceeds that
 * size return WVD_ERR_WORKSPACE before anything is launched (the [1,384,4,44,78] block needs
 * 21.1 MB). Nothing in the scratch needs to start at zero: every byte a call reads it wrote
 * first in the same call. All calls on one GPU share its scratch: calls that may overlap in
 * time on that GPU (other streams, other threads) race; order them on one stream. */
size_t wvd_resblock_noalloc_max_bytes(void);
wvd_status wvd_resblock_noalloc(const wvd_tensor* x, const wvd_resblock_weights* wts, float eps,
                                const wvd_tensor* hist1, const wvd_tensor* hist2, wvd_tensor* y,
                                wvd_tensor* hist1_out, wvd_tensor* hist2_out, wvd_stream stream);

/* ============================================================================================
 * wvd_upsample - 2x upsampling steps (the page's upsample3d / upsample2d parts).
 *  spatial: per frame, nearest x2 in h and w then a 3x3 conv2d C -> C (zero pad 1) + bias;
 *           `spatial` is packed with WVD_PACK_PHASE2X and runs as four phase convolutions.
 *  temporal: a causal (3,1,1) conv C -> 2C (+bias); its output channel c becomes frame 2t and
 *           channel C + c frame 2t + 1. With `first` set (the chunk holding latent frame 0) the
 *           first input frame passes through as one output frame and the conv runs on the frames
 *           after it, with no history ("The first latent frame yields one frame").
 *  order: WVD_TIME_FIRST (the decoder's order) or WVD_SPATIAL_FIRST. Either step may be off
 *  (null weights). time_hist / time_hist_out: as hist / hist_out of wvd_causal_conv3d for the
 *  time conv's input. x, y: bf16 NTHWC. Workspace: wvd_upsample_workspace_bytes(...).
 * ========================================================================================== */
typedef enum { WVD_TIME_FIRST = 0, WVD_SPATIAL_FIRST = 1 } wvd_upsample_order;
size_t wvd_upsample_workspace_bytes(int c, int t, int h, int w, int spatial, int temporal, int order);
wvd_status wvd_upsample(const wvd_tensor* x, const void* spatial, const float* spatial_bias, const void* temporal,
                        const float* temporal_bias, int order, int first, const wvd_tensor* time_hist,
                        wvd_tensor* y, wvd_tensor* time_hist_out, void* ws, size_t ws_bytes, wvd_stream stream);

/* ============================================================================================
 * The whole decoder, streamed in chunks of latent frames with an explicit cache handle
 * (the page's decode and decode_chunk functions and its part list; its "Causal caches" part for
 * what the cache carries). The descriptor describes the synthetic decoder (the real topology's
 * switches all 0) or the real Wan2.2 TI2V-5B topology: post_quant_conv, mid-block attention
 * (base channels a multiple of 32, latent h*w a multiple of 8), stages without the spatial step
 * (and then without a time step or DupUp3D), DupUp3D (out * ft * 4 a multiple of the stage's
 * input channels), a head of colours * patch^2 channels with unpatchify and clamp. The RMS norm
 * is gamma * x / sqrt(mean_c x^2 + eps) throughout; a tiny eps (1e-27) gives the page's
 * x / max(||x||, 1e-12) * sqrt(C) * gamma for every position with a norm above 1e-12. Channels
 * up to 2048. wvd_decoder_param_count returns -1 and wvd_last_error() says why for a
 * descriptor outside these bounds.
 * ========================================================================================== */
#define WVD_MAX_STAGES 8
typedef struct {
  int z_channels;                     /* latent channels (48) */
  int base_channels;                  /* conv_in output and mid blocks (384) */
  int n_stages;                       /* up stages (4) */
  int stage_channels[WVD_MAX_STAGES]; /* (384, 384, 192, 96) */
  int stage_temporal[WVD_MAX_STAGES]; /* time x2 on the stage (1, 1, 0, 0) */
  int mid_resblocks;                  /* residual blocks after conv_in (2) */
  int stage_resblocks;                /* residual blocks per stage (2) */
  int out_channels;                   /* conv_out channels: video colours (3), times patch^2 */
  float eps;                          /* RMS norm epsilon (1e-6) */
  int latent_h, latent_w;             /* latent frame size (44, 78) */
  /* The real Wan2.2 TI2V-5B decoder's parts (the page's part list; all 0 in the synthetic one): */
  int post_quant;                     /* a 1x1x1 conv z -> z in front of conv_in */
  int mid_attention;                  /* single-head attention over each frame after mid block 0 */
  int stage_no_spatial[WVD_MAX_STAGES]; /* 1: the stage has no nearest x2 + 3x3 step */
  int stage_dup[WVD_MAX_STAGES];      /* 1: + DupUp3D of the stage's input after its upsampling */
  int patch;                          /* unpatchify patch p (0 or 1: none); out_channels = 3 p^2 */
  int clamp;                          /* clamp the video to [-1, 1] */
} wvd_decoder_desc;

/* Parameters, in the canonical order (execution order). For index i: its name (e.g.
 * "up.2.res.0.shortcut.weight"), its number of dims and shape. */
int wvd_decoder_param_count(const wvd_decoder_desc* d);
wvd_status wvd_decoder_param_info(const wvd_decoder_desc* d, int index, const char** name, int* ndim,
                                  int64_t shape[5]);
/* Pack every parameter (fp32 device tensors in canonical order) into one device blob. */
size_t wvd_decoder_packed_bytes(const wvd_decoder_desc* d);
wvd_status wvd_decoder_pack(const wvd_decoder_desc* d, const float* const* params, void* packed, wvd_stream stream);

/* The cache: every causal conv's two-frame history, in caller-owned device storage, twice (the
 * current history and the next one: the launch of a chunk's conv that reads a slot's current
 * history also copies the conv's input frames into the slot's other half). */
typedef struct wvd_cache_s* wvd_cache;
size_t wvd_cache_bytes(const wvd_decoder_desc* d);
wvd_status wvd_cache_init(const wvd_decoder_desc* d, void* storage, wvd_cache* out); /* empty history */
wvd_status wvd_cache_reset(wvd_cache c);  /* forget the history: the next chunk must be first */
void wvd_cache_destroy(wvd_cache c);      /* frees the host struct only */
int64_t wvd_cache_next_latent(wvd_cache c); /* latent frames consumed so far */

/* Workspace for chunks of up to `max_latent_frames` latent frames. */
size_t wvd_decode_workspace_bytes(const wvd_decoder_desc* d, int max_latent_frames);

/* Decode one chunk. z: bf16 [1, z_channels, n, latent_h, latent_w], NTHWC or NCTHW. `first`:
 * the chunk holds latent frame 0 (the cache must be empty: fresh or reset); with
 * first_frame_rule set, that frame yields one video frame and the others four, else every
 * latent frame yields 2^(temporal stages) frames. video: bf16 NCTHW [1, out_channels, F,
 * latent_h * 2^n_stages, latent_w * 2^n_stages] (the whole video); the chunk's frames are written
 * from frame_offset on. Returns WVD_ERR_STATE if `first` does not match the cache (first with a
 * used cache, or not first with an empty one), or if frame_offset is not where the previous
 * chunk ended. */
wvd_status wvd_decode_chunk(const wvd_decoder_desc* d, const void* packed, wvd_cache cache, const wvd_tensor* z,
                            int first, int first_frame_rule, wvd_tensor* video, int64_t frame_offset, void* ws,
                            size_t ws_bytes, wvd_stream stream);
/* Video frames a chunk of n latent frames produces. */
int64_t wvd_chunk_video_frames(const wvd_decoder_desc* d, int64_t n, int first, int first_frame_rule);

/* Per-level pass sizes (the FastVideo compare page's suggestion to run many frames through the
 * small early levels and few through the large late ones, section "Memory"): decode one chunk of
 * n latent frames like wvd_decode_chunk, but with 0 < high_latent_frames < n the stages after
 * the last temporal upsample and the head run in sub-passes of high_latent_frames latent frames
 * (the last one shorter), each with the history the previous one left. The video is bit-for-bit
 * the same as with wvd_decode_chunk; the early stages get n frames' worth of work per launch,
 * while the memory of the late stages is bounded by high_latent_frames.
 * high_latent_frames = 0 or >= n: one pass (wvd_decode_chunk). The workspace comes from
 * wvd_decode_workspace_bytes_split(d, n, high_latent_frames); same errors as wvd_decode_chunk,
 * and WVD_ERR_ARG for a negative high_latent_frames. */
size_t wvd_decode_workspace_bytes_split(const wvd_decoder_desc* d, int max_latent_frames, int high_latent_frames);
wvd_status wvd_decode_chunk_split(const wvd_decoder_desc* d, const void* packed, wvd_cache cache, const wvd_tensor* z,
                                  int first, int first_frame_rule, wvd_tensor* video, int64_t frame_offset,
                                  int high_latent_frames, void* ws, size_t ws_bytes, wvd_stream stream);

/* ============================================================================================
 * Kernel timing (measurement support): when enabled, the library records a HIP event pair
 * around every launch of the matrix-core convolution kernel (and of the memory-bound kernels) on
 * the launch stream and sums the elapsed times and the algorithmic FLOPs (bytes) per kernel
 * configuration (kind). wvd_timing_read
 * synchronises the events. Not for use while another thread launches.
 * ========================================================================================== */
wvd_status wvd_timing_enable(int on);
wvd_status wvd_timing_reset(void);
/* For configuration index i (0..count-1): a name, the launch count, the summed milliseconds and
 * the summed algorithmic FLOPs (2*M*N*K with the real, unpadded sizes). Returns the count of
 * configurations when name is null. */
int wvd_timing_read(int i, const char** name, int64_t* launches, double* ms, double* flops);
/* Launch i (0-based, in launch order) since the last reset: its configuration index, milliseconds,
 * algorithmic FLOPs and problem shape {T, H, W, Ci, N, taps, phases, history frames, input frames
 * copied into a cache slot as side work, 1 if it reads a residual}. Returns the number of
 * recorded launches (call with i = -1 to count). */
int wvd_timing_launch(int i, int* config, double* ms, double* flops, int shape[10]);
/* The memory-bound kernels (channel RMS norm + SiLU, the head's tap stencil, the latent layout
 * conversion), timed the same way: for kind i (0..count-1) a name, the launch count, the summed
 * milliseconds and the summed algorithmic bytes (every input element read once, every output
 * element written once). Returns the count of kinds when name is null. */
int wvd_timing_read_mem(int i, const char** name, int64_t* launches, double* ms, double* bytes);
/* Testing and tuning support: run every following matrix-core convolution launch with
 * configuration `config` (an index of wvd_timing_read), or with the automatic choice again
 * when config is -1. A launch the forced configuration cannot run (a halo-tile configuration on
 * a convolution without 3x3 spatial taps, or a channel tile narrower than a fused norm needs)
 * fails with WVD_ERR_UNSUPPORTED. WVD_ERR_ARG for an index out of range. Process-wide; not for
 * use while another thread launches. */
wvd_status wvd_conv_force_config(int config);
/* Testing support: cap the workgroups of every following halo-tile (LDS-DMA) convolution launch
 * that walks several tiles per workgroup (those without a fused norm) at n, rounded down to a
 * multiple of 8 and at least 8, so that each workgroup walks a longer run of tiles; 0 restores
 * the default (one workgroup per resident slot). Results are the same for any n. WVD_ERR_ARG for
 * n < 0. Process-wide; not for use while another thread launches. */
wvd_status wvd_conv_max_workgroups(int n);
/* Tuning: with on != 0 (the default), wvd_decode_chunk applies each residual block's norm1 +
 * SiLU in the epilogue of the conv that produces its input, where one workgroup holds every
 * channel (the previous block's conv2 up to 192 channels, an x2 upsample of 97-192 channels not
 * followed by a DupUp3D add): that conv stores both its output and the next block's activated
 * input, and the standalone norm pass goes (the page's merge of the next conv's norm into the
 * producing epilogue, "The merges"). With on == 0 every norm1 is a separate pass. The two videos
 * differ by rounding only (the fused norm reads the unrounded fp32 output); either way decodes
 * are bitwise independent of the pass size. Process-wide; not for use while another thread
 * decodes. */
wvd_status wvd_decode_fuse_norm1(int on);
/* Tuning: with on != 0 (the default), when an x2 upsample of 192 channels stores both its output
 * and the next block's activated input (wvd_decode_fuse_norm1) and that block starts with a 1x1
 * shortcut to 96 channels (the page's residual block part: cin != cout), the upsample's epilogue
 * applies the shortcut (plus its bias) to its own output, rounded to bf16 as the stored output
 * would be, and stores that product instead of the output, which the shortcut alone would read;
 * the shortcut pass goes. With on == 0 the output is stored and the shortcut runs as its own
 * pass. The two videos differ by the summation order of the shortcut only; either way decodes
 * are bitwise independent of the pass size. Process-wide; not for use while another thread
 * decodes. */
wvd_status wvd_decode_fuse_shortcut(int on);
/* Tuning: with on != 0 (the default), a residual block whose channel count changes from 384 to
 * at most 192 (a multiple of 32) takes its norm1 + SiLU and its 1x1 shortcut (the page's residual
 * block: the input feeds both the normalised branch and, when cin != cout, the shortcut) from
 * one read of its input, in one kernel, instead of in two passes that each read it; both outputs
 * are bitwise the same either way. Used by wvd_resblock, wvd_resblock_noalloc and the decode
 * calls when the weights, bias and gamma are 16-byte aligned. Process-wide; not for use while
 * another thread runs those calls. */
wvd_status wvd_fuse_norm_shortcut(int on);
/* Memory option: with on != 0, a decoder whose last stage is a spatial x2 upsample (no time
 * step, no DupUp3D) of 65-96 channels and whose head is conv_out to at most 3 colours (no
 * unpatchify or clamp) runs that upsample, norm_out + SiLU and the head as one kernel per pass:
 * the activated last-level tensor (the largest of the decode) is never written, and the head's
 * causal cache holds, instead of its last two input frames, the partial sums of the two output
 * frames after the pass (fp32, 3 x H x W each): at 704x1248, 650 MB less cache and 0.6 GiB less
 * peak memory, but about 3 % slower (the fused kernel runs one workgroup per CU). With on == 0
 * (the default) the upsample writes the activated tensor and the head reads it (in frame
 * sub-passes). The cache layout follows the
 * switch: wvd_cache_bytes, wvd_cache_init and the workspace sizes read it, and a decode whose
 * switch differs from the one its cache was made with fails with WVD_ERR_STATE. The two videos
 * differ by rounding only; either way decodes are bitwise independent of the pass size.
 * Process-wide; not for use while another thread decodes. */
wvd_status wvd_decode_fuse_head(int on);
/* Measurement support: copy `bytes` (a multiple of 16; src and dst 16-byte aligned, device
 * memory, not overlapping) with the convolution kernels' own load path: buffer loads that write
 * 16 bytes per lane straight into LDS, read back and stored with 16-byte global stores. The
 * hardware byte counters of this copy, whose true traffic is known, give the factor that turns
 * the counters of the convolution kernels into bytes. WVD_ERR_ALIGN / WVD_ERR_ARG on bad
 * arguments, before any launch. */
wvd_status wvd_calib_dma_copy(const void* src, void* dst, size_t bytes, wvd_stream stream);

#ifdef __cplusplus
}
#endif
#endif /* WVD_H */
