// C ABI of libwvd: validation, dispatch, the layer drivers (residual block, upsampling), the
// decoder's weight packing, cache handle and chunk driver, and kernel timing.
//
// The decode follows the reference decoder printed on the FastVideo compare page "[perf] PAN2
// sampling: Wan2.2 VAE decode kernel, split decode, fused DiT kernels" (its decode_chunk,
// up_block, residual_block, cached_conv and causal_conv functions, and the docstring's "Causal
// caches" and "The first latent frame yields one frame" parts), in the synthetic topology of
// wvd_decoder_desc. All device memory comes from the caller.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <new>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/wvd.h"
#include "common.h"

using namespace wvd;

namespace {

thread_local std::string g_err;

wvd_status fail(wvd_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

wvd_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return WVD_OK;
  return fail(WVD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define WVD_TRY(expr)                  \
  do {                                 \
    const wvd_status _st = (expr);     \
    if (_st != WVD_OK) return _st;     \
  } while (0)

#define WVD_HIP(expr, what)                                   \
  do {                                                        \
    const hipError_t _e = (expr);                             \
    if (_e != hipSuccess) return hip_status(_e, what);        \
  } while (0)

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int64_t numel(const wvd_tensor* t) { return t->n * t->c * t->t * t->h * t->w; }
size_t elem_size(int dtype) { return dtype == WVD_BF16 ? 2 : 4; }

// Checks a tensor descriptor; `dtype`/`layout` -1 accept any.
wvd_status check_tensor(const wvd_tensor* t, const char* name, int dtype, int layout, bool allow_empty_t) {
  if (!t) return fail(WVD_ERR_ARG, "%s is null", name);
  if (t->n != 1) return fail(WVD_ERR_SHAPE, "%s: batch must be 1 (got %lld)", name, (long long)t->n);
  if (t->c <= 0 || t->h <= 0 || t->w <= 0 || t->t < 0 || (!allow_empty_t && t->t == 0))
    return fail(WVD_ERR_SHAPE, "%s: invalid sizes [%lld,%lld,%lld,%lld,%lld]", name, (long long)t->n,
                (long long)t->c, (long long)t->t, (long long)t->h, (long long)t->w);
  if (t->dtype != WVD_F32 && t->dtype != WVD_BF16) return fail(WVD_ERR_DTYPE, "%s: unknown dtype %d", name, t->dtype);
  if (t->layout != WVD_NCTHW && t->layout != WVD_NTHWC)
    return fail(WVD_ERR_LAYOUT, "%s: unknown layout %d", name, t->layout);
  if (dtype >= 0 && t->dtype != dtype)
    return fail(WVD_ERR_DTYPE, "%s: expected %s", name, dtype == WVD_BF16 ? "bf16" : "fp32");
  if (layout >= 0 && t->layout != layout)
    return fail(WVD_ERR_LAYOUT, "%s: expected %s", name, layout == WVD_NTHWC ? "NTHWC" : "NCTHW");
  if (numel(t) > 0 && !t->data) return fail(WVD_ERR_ARG, "%s: null data", name);
  if (t->data && !aligned16(t->data)) return fail(WVD_ERR_ALIGN, "%s: data not 16-byte aligned", name);
  if (numel(t) * (int64_t)t->c > ((int64_t)1 << 62)) return fail(WVD_ERR_SHAPE, "%s: too large", name);
  return WVD_OK;
}

bool same_grid(const wvd_tensor* a, const wvd_tensor* b) { return a->h == b->h && a->w == b->w; }

// Whether the byte ranges of two tensors overlap (empty tensors overlap nothing).
bool overlaps(const wvd_tensor* a, const wvd_tensor* b) {
  if (!a || !b || numel(a) == 0 || numel(b) == 0) return false;
  const char* a0 = (const char*)a->data;
  const char* b0 = (const char*)b->data;
  const char* a1 = a0 + numel(a) * elem_size(a->dtype);
  const char* b1 = b0 + numel(b) * elem_size(b->dtype);
  return a0 < b1 && b0 < a1;
}

// ------------------------------------------------------------------------------------------
// Timing of the matrix-core conv launches.
// ------------------------------------------------------------------------------------------
struct TimingRecord {
  int config;  // conv configuration, or -1 for a memory-bound kernel
  int mem;     // MemKind of a memory-bound kernel, or -1
  hipEvent_t start, stop;
  double flops;  // conv: algorithmic FLOPs; memory-bound kernel: algorithmic bytes
  int shape[10];  // T, H, W, Ci, N, taps, phases, Th, cache frames copied as side work, residual read
};
// The memory-bound kernels of the path, timed like the convs (algorithmic bytes: every input
// element read once, every output element written once).
enum MemKind {
  MEM_NORM_SILU = 0,
  MEM_HEAD_STENCIL = 1,
  MEM_CONVERT = 2,
  MEM_HEAD_FUSED = 3,
  MEM_HEAD_STREAM = 4,
  MEM_ATTN = 5,     // the attention's softmax and value transpose
  MEM_DUP = 6,      // the DupUp3D add
  MEM_UNPATCH = 7,  // unpatchify (+ clamp) into the video
  MEM_WINO_IN = 8,  // the Winograd input transform
  MEM_WINO_OUT = 9, // the Winograd output transform
  MEM_NORM_SC = 10, // a residual block's norm1 + SiLU and 1x1 shortcut from one read of its input
  MEM_KINDS = 11
};
const char* const kMemKindNames[MEM_KINDS] = {"norm_silu", "head_stencil", "convert", "head_fused", "head_stream",
                                              "attn_softmax_transpose", "dup_add", "unpatchify", "winograd_in",
                                              "winograd_out", "norm_shortcut"};
struct LaunchRecord {
  int config;
  float ms;
  double flops;
  int shape[10];
};
struct TimingState {
  std::mutex mu;
  bool on = false;
  std::vector<TimingRecord> pending;
  std::vector<hipEvent_t> pool;
  std::vector<int64_t> launches;
  std::vector<double> ms, flops;
  int64_t mem_launches[MEM_KINDS] = {};
  double mem_ms[MEM_KINDS] = {}, mem_bytes[MEM_KINDS] = {};
  std::vector<LaunchRecord> log;  // every timed conv launch since the last reset
} g_timing;

hipEvent_t pooled_event() {
  if (!g_timing.pool.empty()) {
    hipEvent_t e = g_timing.pool.back();
    g_timing.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Configuration forced by wvd_conv_force_config (-1: automatic choice) and the workgroup cap of
// wvd_conv_max_workgroups (0: none).
std::atomic<int> g_force_config{-1};
std::atomic<int> g_max_workgroups{0};

wvd_status run_conv(const ConvProblem& p, hipStream_t s, double flops) {
  const bool timed = g_timing.on;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (timed) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    e0 = pooled_event();
    e1 = pooled_event();
    if (!e0 || !e1) return fail(WVD_ERR_HIP, "hipEventCreate failed");
    WVD_HIP(hipEventRecord(e0, s), "hipEventRecord");
  }
  int cfg = -1;
  const hipError_t le = launch_conv_mfma(p, s, &cfg, g_force_config.load(), g_max_workgroups.load());
  if (le == hipErrorNotSupported) return fail(WVD_ERR_UNSUPPORTED, "forced conv configuration cannot run this problem");
  WVD_HIP(le, "conv_mfma launch");
  if (timed) {
    WVD_HIP(hipEventRecord(e1, s), "hipEventRecord");
    std::lock_guard<std::mutex> lk(g_timing.mu);
    const int copied = (int)((p.copy.bytes[0] + p.copy.bytes[1]) / std::max<int64_t>(1, (int64_t)p.H * p.W * p.Ci * 2));
    TimingRecord r{cfg, -1, e0, e1, flops, {p.T, p.H, p.W, p.Ci, p.N, p.ntaps, p.phases, p.Th, copied, p.res ? 1 : 0}};
    g_timing.pending.push_back(r);
  }
  return WVD_OK;
}

// A memory-bound launch (`launch` returns a hipError_t), timed when timing is on.
template <class F>
wvd_status run_mem(int kind, double bytes, hipStream_t s, const char* what, F&& launch) {
  const bool timed = g_timing.on;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (timed) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    e0 = pooled_event();
    e1 = pooled_event();
    if (!e0 || !e1) return fail(WVD_ERR_HIP, "hipEventCreate failed");
    WVD_HIP(hipEventRecord(e0, s), "hipEventRecord");
  }
  WVD_HIP(launch(), what);
  if (timed) {
    WVD_HIP(hipEventRecord(e1, s), "hipEventRecord");
    std::lock_guard<std::mutex> lk(g_timing.mu);
    g_timing.pending.push_back(TimingRecord{-1, kind, e0, e1, bytes, {}});
  }
  return WVD_OK;
}

// Channel RMS norm (+ SiLU) over P positions of C channels (NTHWC bf16): reads x and gamma,
// writes y.
wvd_status run_norm(const bf16_t* x, const float* gamma, float eps, int silu, bf16_t* y, int64_t P, int C,
                    hipStream_t s) {
  return run_mem(MEM_NORM_SILU, 4.0 * (double)P * C + 4.0 * C, s, "norm launch",
                 [&] { return launch_norm_silu(x, gamma, eps, silu, y, P, C, s); });
}

std::atomic<int> g_fuse_norm_sc{1};  // wvd_fuse_norm_shortcut

// Whether a residual block's norm1 and shortcut of cin -> cout channels run as one pass.
bool norm_sc_fused(int cin, int cout, const void* wsc, const float* bsc, const float* gamma) {
  return g_fuse_norm_sc.load() && cin != cout && norm_shortcut_supported(cin, cout) && aligned16(wsc) &&
         aligned16(bsc) && aligned16(gamma);
}

// norm1 + SiLU of x into a and the 1x1 shortcut of x into sc, one read of x: reads x, the packed
// weight and gamma, writes both outputs.
wvd_status run_norm_sc(const bf16_t* x, const float* gamma, float eps, bf16_t* a, const void* wsc, int cout,
                       const float* bsc, bf16_t* sc, int64_t P, int C, hipStream_t s) {
  const double bytes = 2.0 * P * C * 2.0 + 2.0 * (double)P * cout + 2.0 * (double)cout * C + 4.0 * C;
  return run_mem(MEM_NORM_SC, bytes, s, "norm and shortcut launch", [&] {
    return launch_norm_shortcut(x, P, C, gamma, eps, a, (const bf16_t*)wsc, cout, bsc, sc, s);
  });
}

// ------------------------------------------------------------------------------------------
// Convolution problems
// ------------------------------------------------------------------------------------------
int64_t packed_elems(int co, int ci, int taps, int phases) {
  return (int64_t)phases * round_up(co, 32) * taps * round_up(ci, 32);
}

// A plain causal conv on NTHWC bf16: y [T][H][W][Co] (+ residual).
ConvProblem plain_problem(const bf16_t* x, const bf16_t* hist, int T, int H, int W, int Ci, int Th,
                          const void* wpk, int co, int kt, int kh, int kw, const float* bias, bf16_t* y,
                          const bf16_t* res) {
  ConvProblem p;
  memset(&p, 0, sizeof(p));
  p.x = x;
  p.hist = hist;
  p.T = T;
  p.H = H;
  p.W = W;
  p.Ci = Ci;
  p.Th = hist ? Th : 0;
  p.wpk = (const bf16_t*)wpk;
  p.ntaps = kt * kh * kw;
  p.Cip = (int)round_up(Ci, 32);
  p.Npad = (int)round_up(co, 32);
  p.phases = 1;
  p.kt = kt;
  p.kh = kh;
  p.kw = kw;
  p.N = co;
  p.bias = bias;
  p.y = y;
  p.res = res;
  p.To = T;
  p.Ho = H;
  p.Wo = W;
  p.nsplit = co;
  p.fbase = 0;
  p.fmul = 1;
  p.fstride = 1;
  p.hmul = 1;
  p.wmul = 1;
  return p;
}

double conv_flops(int64_t M, int N, int64_t K) { return 2.0 * (double)M * (double)N * (double)K; }

// Causal time conv C -> 2C whose output channel c goes to frame fbase + 2t and C + c to
// fbase + 2t + 1 of y [To][H][W][C].
wvd_status run_time_conv(const bf16_t* x, const bf16_t* hist, int T, int H, int W, int C, int Th, const void* wpk,
                         const float* bias, bf16_t* y, int To, int fbase, hipStream_t s) {
  ConvProblem p = plain_problem(x, hist, T, H, W, C, Th, wpk, 2 * C, 3, 1, 1, bias, y, nullptr);
  p.To = To;
  p.nsplit = C;
  p.fmul = 2;
  p.fbase = fbase;
  return run_conv(p, s, conv_flops((int64_t)T * H * W, 2 * C, 3LL * C));
}

// Nearest x2 + 3x3 conv as four phase convs: x [T][H][W][C] -> y [T][2H][2W][C]; with norm_gamma,
// y is SiLU(RMS norm) of the upsampled tensor (fused in the epilogue).
// sc_w / sc_b / sc_co / y_sc: the dual store's shortcut product in place of y_pre (ConvProblem::y_sc).
wvd_status run_phase_conv(const bf16_t* x, int T, int H, int W, int C, const void* wpk, const float* bias, bf16_t* y,
                          hipStream_t s, const float* norm_gamma = nullptr, float norm_eps = 0.0f,
                          bf16_t* y_pre = nullptr, const void* sc_w = nullptr, const float* sc_b = nullptr,
                          int sc_co = 0, bf16_t* y_sc = nullptr) {
  ConvProblem p = plain_problem(x, nullptr, T, H, W, C, 0, wpk, C, 1, 1, 1, bias, y, nullptr);
  p.norm_gamma = norm_gamma;
  p.y_pre = y_pre;
  p.sc_w = (const bf16_t*)sc_w;
  p.sc_b = sc_b;
  p.sc_co = sc_co;
  p.sc_wrow = (int)round_up(C, 32);
  p.y_sc = y_sc;
  p.norm_eps = norm_eps;
  p.norm_silu = 1;
  p.ntaps = 4;
  p.phases = 4;
  p.kt = 1;
  p.kh = 2;
  p.kw = 2;
  p.Ho = 2 * H;
  p.Wo = 2 * W;
  p.hmul = 2;
  p.wmul = 2;
  const int64_t P = (int64_t)T * H * W * 4;
  return run_conv(p, s, conv_flops(P, C, 4LL * C) + (y_sc ? conv_flops(P, sc_co, C) : 0.0));
}

// History a conv leaves (the page's cached_conv rule), copied into a separate tensor.
// frame_bytes: bytes of one frame (NTHWC) of the conv input.
wvd_status copy_history_out(const void* x, int T, const void* hist, int Th, void* out, size_t frame_bytes,
                            hipStream_t s) {
  if (T >= 2) {
    WVD_HIP(hipMemcpyAsync(out, (const char*)x + (size_t)(T - 2) * frame_bytes, 2 * frame_bytes,
                           hipMemcpyDeviceToDevice, s),
            "history copy");
  } else if (T == 1) {
    if (Th >= 1) {
      WVD_HIP(hipMemcpyAsync(out, (const char*)hist + (size_t)(Th - 1) * frame_bytes, frame_bytes,
                             hipMemcpyDeviceToDevice, s),
              "history copy");
      WVD_HIP(hipMemcpyAsync((char*)out + frame_bytes, x, frame_bytes, hipMemcpyDeviceToDevice, s), "history copy");
    } else {
      WVD_HIP(hipMemcpyAsync(out, x, frame_bytes, hipMemcpyDeviceToDevice, s), "history copy");
    }
  } else if (Th > 0) {
    WVD_HIP(hipMemcpyAsync(out, hist, (size_t)Th * frame_bytes, hipMemcpyDeviceToDevice, s), "history copy");
  }
  return WVD_OK;
}

int history_frames_after(int T, int Th) {
  if (T >= 2) return 2;
  if (T == 1) return Th >= 1 ? 2 : 1;
  return Th;
}

// Cache slots are double-buffered: two halves of [2][frame], `half` naming the one that holds
// the current history (`valid` frames, right-aligned). The update writes the next history (the
// page's cached_conv rule: the last two input frames, or the old last frame and a one-frame
// input) into the other half, so it can run as side work of the very launch that still reads
// the current one (`job`, zero bytes when there is nothing to copy); `half` and `valid` become
// the slot's state once that launch is enqueued.
void slot_update_job(char* slot, int& half, int& valid, const void* x, int T, size_t frame_bytes, CopyJob& job) {
  memset(&job, 0, sizeof(job));
  const char* cur = slot + (size_t)half * 2 * frame_bytes;
  char* nxt = slot + (size_t)(half ^ 1) * 2 * frame_bytes;
  if (T >= 2) {
    job.src[0] = (const char*)x + (size_t)(T - 2) * frame_bytes;
    job.dst[0] = nxt;
    job.bytes[0] = (int64_t)(2 * frame_bytes);
    valid = 2;
  } else if (T == 1) {
    if (valid >= 1) {
      job.src[0] = cur + frame_bytes;
      job.dst[0] = nxt;
      job.bytes[0] = (int64_t)frame_bytes;
    }
    job.src[1] = x;
    job.dst[1] = nxt + frame_bytes;
    job.bytes[1] = (int64_t)frame_bytes;
    valid = valid >= 1 ? 2 : 1;
  } else {
    return;
  }
  half ^= 1;
}

}  // namespace

// ==============================================================================================
// Basic entry points
// ==============================================================================================
extern "C" const char* wvd_last_error(void) { return g_err.c_str(); }
extern "C" int wvd_abi_version(void) { return WVD_ABI_VERSION; }

extern "C" wvd_status wvd_convert(const wvd_tensor* x, wvd_tensor* y, wvd_stream stream) {
  WVD_TRY(check_tensor(x, "x", -1, -1, true));
  WVD_TRY(check_tensor(y, "y", -1, -1, true));
  if (x->c != y->c || x->t != y->t || x->h != y->h || x->w != y->w)
    return fail(WVD_ERR_SHAPE, "convert: x and y sizes differ");
  if (x->data == y->data && numel(x) > 0) return fail(WVD_ERR_ARG, "convert: x and y must not overlap");
  return hip_status(launch_convert(x->data, x->dtype == WVD_BF16, x->layout == WVD_NCTHW, y->data, y->dtype == WVD_BF16,
                                   y->layout == WVD_NCTHW, (int)x->c, (int)x->t, (int)x->h, (int)x->w,
                                   (hipStream_t)stream),
                    "convert launch");
}

extern "C" size_t wvd_conv_packed_bytes(int co, int ci, int kt, int kh, int kw, int mode) {
  if (co <= 0 || ci <= 0) return 0;
  if (mode == WVD_PACK_PHASE2X) return (size_t)packed_elems(co, ci, 4, 4) * 2;
  if (mode != WVD_PACK_CONV || kt <= 0 || kh <= 0 || kw <= 0 || kt % 2 == 0 || kh % 2 == 0 || kw % 2 == 0 ||
      kt * kh * kw > 27)
    return 0;
  return (size_t)packed_elems(co, ci, kt * kh * kw, 1) * 2;
}

extern "C" wvd_status wvd_conv_pack(const void* w_raw, int w_dtype, int co, int ci, int kt, int kh, int kw, int mode,
                                    void* packed, wvd_stream stream) {
  if (!w_raw || !packed) return fail(WVD_ERR_ARG, "conv_pack: null pointer");
  if (w_dtype != WVD_F32 && w_dtype != WVD_BF16) return fail(WVD_ERR_DTYPE, "conv_pack: weight dtype");
  if (co <= 0 || ci <= 0) return fail(WVD_ERR_SHAPE, "conv_pack: channels must be positive");
  if (!aligned16(packed)) return fail(WVD_ERR_ALIGN, "conv_pack: packed buffer not 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const int npad = (int)round_up(co, 32), cip = (int)round_up(ci, 32);
  if (mode == WVD_PACK_PHASE2X) {
    if (kt != 1 || kh != 3 || kw != 3) return fail(WVD_ERR_SHAPE, "conv_pack: phase packing needs a 1x3x3 kernel");
    return hip_status(launch_pack_phase2x(w_raw, w_dtype == WVD_BF16, co, ci, npad, cip, (bf16_t*)packed, s),
                      "pack launch");
  }
  if (mode != WVD_PACK_CONV) return fail(WVD_ERR_ARG, "conv_pack: unknown mode %d", mode);
  if (kt <= 0 || kh <= 0 || kw <= 0 || kt % 2 == 0 || kh % 2 == 0 || kw % 2 == 0 || kt * kh * kw > 27)
    return fail(WVD_ERR_UNSUPPORTED, "conv_pack: kernel sizes must be odd with at most 27 taps");
  return hip_status(launch_pack_conv(w_raw, w_dtype == WVD_BF16, co, ci, kt * kh * kw, npad, cip, (bf16_t*)packed, s),
                    "pack launch");
}

extern "C" wvd_status wvd_causal_conv3d(const wvd_tensor* x, const void* w, int co, int kt, int kh, int kw,
                                        const float* bias, const wvd_tensor* hist, const wvd_tensor* residual,
                                        wvd_tensor* y, wvd_tensor* hist_out, wvd_stream stream) {
  WVD_TRY(check_tensor(x, "x", -1, -1, true));
  WVD_TRY(check_tensor(y, "y", x->dtype, x->layout, true));
  if (!w) return fail(WVD_ERR_ARG, "weights are null");
  if (co <= 0 || kt <= 0 || kh <= 0 || kw <= 0 || kt % 2 == 0 || kh % 2 == 0 || kw % 2 == 0 || kt * kh * kw > 27)
    return fail(WVD_ERR_UNSUPPORTED, "kernel sizes must be odd with at most 27 taps, co > 0");
  if (y->c != co || y->t != x->t || !same_grid(x, y)) return fail(WVD_ERR_SHAPE, "y must be [1, co, T, H, W] of x");
  const int P = 2 * (kt / 2);
  int Th = 0;
  if (hist) {
    WVD_TRY(check_tensor(hist, "hist", x->dtype, x->layout, true));
    if (hist->c != x->c || !same_grid(hist, x)) return fail(WVD_ERR_SHAPE, "hist must match x in c, h, w");
    if (hist->t > P) return fail(WVD_ERR_SHAPE, "hist has %lld frames, the conv takes at most %d", (long long)hist->t, P);
    Th = (int)hist->t;
  }
  if (hist_out) {
    WVD_TRY(check_tensor(hist_out, "hist_out", x->dtype, x->layout, true));
    if (hist_out->c != x->c || !same_grid(hist_out, x)) return fail(WVD_ERR_SHAPE, "hist_out must match x in c, h, w");
    const int want = history_frames_after((int)x->t, Th);
    if (hist_out->t != want) return fail(WVD_ERR_SHAPE, "hist_out must have %d frames", want);
    if (hist && hist_out->data == hist->data && want > 0) return fail(WVD_ERR_ARG, "hist_out may not alias hist");
    if (x->layout != WVD_NTHWC) return fail(WVD_ERR_LAYOUT, "hist_out needs NTHWC tensors");
  }
  // Workgroups read the frames and halo rows of x and hist that other workgroups write in y:
  // an in-place call would race, so y may share no byte with them (nor hist_out with any of them).
  if (overlaps(y, x)) return fail(WVD_ERR_ARG, "y may not overlap x");
  if (overlaps(y, hist)) return fail(WVD_ERR_ARG, "y may not overlap hist");
  if (hist_out && (overlaps(hist_out, x) || overlaps(hist_out, hist) || overlaps(hist_out, y)))
    return fail(WVD_ERR_ARG, "hist_out may not overlap x, hist or y");
  if (!aligned16(w)) return fail(WVD_ERR_ALIGN, "weights not 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const int T = (int)x->t, H = (int)x->h, W = (int)x->w, Ci = (int)x->c;
  if (x->dtype == WVD_F32) {
    if (residual) return fail(WVD_ERR_UNSUPPORTED, "the fp32 path takes no residual");
    if (T > 0)
      WVD_HIP(launch_conv_fp32((const float*)x->data, hist ? (const float*)hist->data : nullptr, (const float*)w, bias,
                               (float*)y->data, Ci, T, H, W, Th, co, kt, kh, kw, x->layout == WVD_NCTHW, s),
              "conv_fp32 launch");
  } else {
    if (x->layout != WVD_NTHWC) return fail(WVD_ERR_LAYOUT, "the bf16 path needs NTHWC tensors");
    if (Ci % 8 != 0) return fail(WVD_ERR_UNSUPPORTED, "bf16 path: input channels must be a multiple of 8");
    if (co % 4 != 0) return fail(WVD_ERR_UNSUPPORTED, "bf16 path: output channels must be a multiple of 4");
    if (residual) {
      WVD_TRY(check_tensor(residual, "residual", WVD_BF16, WVD_NTHWC, true));
      if (residual->c != co || residual->t != x->t || !same_grid(residual, x))
        return fail(WVD_ERR_SHAPE, "residual must have y's shape");
    }
    if ((int64_t)T * H * W >= ((int64_t)1 << 31)) return fail(WVD_ERR_UNSUPPORTED, "too many positions");
    if (T > 0) {
      ConvProblem p = plain_problem((const bf16_t*)x->data, hist ? (const bf16_t*)hist->data : nullptr, T, H, W, Ci,
                                    Th, w, co, kt, kh, kw, bias, (bf16_t*)y->data,
                                    residual ? (const bf16_t*)residual->data : nullptr);
      WVD_TRY(run_conv(p, s, conv_flops((int64_t)T * H * W, co, (int64_t)kt * kh * kw * Ci)));
    }
  }
  if (hist_out)
    WVD_TRY(copy_history_out(x->data, T, hist ? hist->data : nullptr, Th, hist_out->data,
                             (size_t)H * W * Ci * elem_size(x->dtype), s));
  return WVD_OK;
}

// ==============================================================================================
// Winograd F(2x2, 3x3) form of the causal 3x3x3 convolution (winograd.hip)
// ==============================================================================================
namespace {

struct WinoWs {
  size_t u, m, total;  // byte offsets of U [16][Th+T][tH][tW][Ci] bf16 and M [16][T][tH][tW][Co] fp32
};

WinoWs wino_ws(int ci, int co, int64_t t, int64_t th, int64_t h, int64_t w) {
  const int64_t tiles = ((h + 1) / 2) * ((w + 1) / 2);
  WinoWs r;
  r.u = 0;
  r.m = (size_t)round_up(16 * (t + th) * tiles * ci * 2, 256);
  r.total = r.m + (size_t)round_up(16 * t * tiles * co * 4, 256);
  return r;
}

}  // namespace

extern "C" size_t wvd_winograd_packed_bytes(int co, int ci) {
  if (co <= 0 || ci <= 0) return 0;
  return (size_t)packed_elems(co, ci, 3, 16) * 2;
}

extern "C" wvd_status wvd_winograd_pack(const void* w_raw, int w_dtype, int co, int ci, void* packed,
                                        wvd_stream stream) {
  if (!w_raw || !packed) return fail(WVD_ERR_ARG, "winograd_pack: null pointer");
  if (w_dtype != WVD_F32 && w_dtype != WVD_BF16) return fail(WVD_ERR_DTYPE, "winograd_pack: weight dtype");
  if (co <= 0 || ci <= 0) return fail(WVD_ERR_SHAPE, "winograd_pack: channels must be positive");
  if (!aligned16(packed)) return fail(WVD_ERR_ALIGN, "winograd_pack: packed buffer not 16-byte aligned");
  return hip_status(launch_wino_pack(w_raw, w_dtype == WVD_BF16, co, ci, (int)round_up(co, 32), (int)round_up(ci, 32),
                                     (bf16_t*)packed, (hipStream_t)stream),
                    "winograd pack launch");
}

extern "C" size_t wvd_winograd_workspace_bytes(int ci, int co, int t, int th, int h, int w) {
  if (ci <= 0 || co <= 0 || t < 0 || th < 0 || h <= 0 || w <= 0) return 0;
  return wino_ws(ci, co, t, th, h, w).total;
}

extern "C" wvd_status wvd_causal_conv3d_winograd(const wvd_tensor* x, const void* w_packed, int co, const float* bias,
                                                 const wvd_tensor* hist, const wvd_tensor* residual, wvd_tensor* y,
                                                 void* ws, size_t ws_bytes, wvd_stream stream) {
  WVD_TRY(check_tensor(x, "x", WVD_BF16, WVD_NTHWC, true));
  WVD_TRY(check_tensor(y, "y", WVD_BF16, WVD_NTHWC, true));
  if (!w_packed || !aligned16(w_packed)) return fail(WVD_ERR_ALIGN, "winograd: packed weights null or unaligned");
  if (bias && !aligned16(bias)) return fail(WVD_ERR_ALIGN, "winograd: bias not 16-byte aligned");
  const int Ci = (int)x->c, T = (int)x->t, H = (int)x->h, W = (int)x->w;
  if (Ci % 8 != 0 || co <= 0 || co % 4 != 0)
    return fail(WVD_ERR_UNSUPPORTED, "winograd: input channels a multiple of 8, output channels of 4");
  if (y->c != co || y->t != x->t || !same_grid(x, y)) return fail(WVD_ERR_SHAPE, "y must be [1, co, T, H, W] of x");
  int Th = 0;
  if (hist) {
    WVD_TRY(check_tensor(hist, "hist", WVD_BF16, WVD_NTHWC, true));
    if (hist->c != x->c || !same_grid(hist, x) || hist->t > 2) return fail(WVD_ERR_SHAPE, "hist must be [1, ci, <=2, H, W]");
    Th = (int)hist->t;
  }
  if (residual) {
    WVD_TRY(check_tensor(residual, "residual", WVD_BF16, WVD_NTHWC, true));
    if (residual->c != co || residual->t != x->t || !same_grid(residual, x))
      return fail(WVD_ERR_SHAPE, "residual must have y's shape");
  }
  if (overlaps(y, x) || overlaps(y, hist)) return fail(WVD_ERR_ARG, "y may not overlap x or hist");
  const WinoWs wl = wino_ws(Ci, co, T, Th, H, W);
  if (ws_bytes < wl.total) return fail(WVD_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, wl.total);
  if (T == 0) return WVD_OK;
  if (!ws || !aligned16(ws)) return fail(WVD_ERR_ALIGN, "workspace null or not 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const int tH = (H + 1) / 2, tW = (W + 1) / 2;
  const int64_t tiles = (int64_t)tH * tW;
  bf16_t* U = (bf16_t*)((char*)ws + wl.u);
  float* M = (float*)((char*)ws + wl.m);
  const double in_bytes = 2.0 * (T + Th) * H * W * Ci + 2.0 * 16 * (T + Th) * tiles * Ci;
  WVD_TRY(run_mem(MEM_WINO_IN, in_bytes, s, "winograd input transform", [&] {
    return launch_wino_in((const bf16_t*)x->data, hist ? (const bf16_t*)hist->data : nullptr, T, Th, H, W, Ci, U, s);
  }));
  const int64_t u_plane = (int64_t)(T + Th) * tiles * Ci, m_plane = (int64_t)T * tiles * co;
  const int64_t w_plane = packed_elems(co, Ci, 3, 1);
  for (int xi = 0; xi < 16; ++xi) {
    const bf16_t* u = U + xi * u_plane;
    ConvProblem cp = plain_problem(u + (int64_t)Th * tiles * Ci, Th ? u : nullptr, T, tH, tW, Ci, Th,
                                   (const bf16_t*)w_packed + xi * w_plane, co, 3, 1, 1, nullptr, nullptr, nullptr);
    cp.y = M + xi * m_plane;
    cp.y_f32 = 1;
    WVD_TRY(run_conv(cp, s, conv_flops((int64_t)T * tiles, co, 3LL * Ci)));
  }
  const double out_bytes = 4.0 * 16 * T * tiles * co + 2.0 * T * H * W * co * (residual ? 2 : 1);
  return run_mem(MEM_WINO_OUT, out_bytes, s, "winograd output transform", [&] {
    return launch_wino_out(M, T, H, W, co, bias, residual ? (const bf16_t*)residual->data : nullptr, (bf16_t*)y->data,
                           s);
  });
}

extern "C" wvd_status wvd_rmsnorm_silu(const wvd_tensor* x, const float* gamma, float eps, int apply_silu, wvd_tensor* y,
                                       wvd_stream stream) {
  WVD_TRY(check_tensor(x, "x", WVD_BF16, WVD_NTHWC, true));
  WVD_TRY(check_tensor(y, "y", WVD_BF16, WVD_NTHWC, true));
  if (!gamma) return fail(WVD_ERR_ARG, "gamma is null");
  if (x->c != y->c || x->t != y->t || !same_grid(x, y)) return fail(WVD_ERR_SHAPE, "y must have x's shape");
  if (x->c % 8 != 0 || x->c > 2048) return fail(WVD_ERR_UNSUPPORTED, "channels must be a multiple of 8, at most 2048");
  if (!(eps >= 0.0f)) return fail(WVD_ERR_ARG, "eps must be >= 0");
  return run_norm((const bf16_t*)x->data, gamma, eps, apply_silu, (bf16_t*)y->data, x->t * x->h * x->w, (int)x->c,
                  (hipStream_t)stream);
}

// ==============================================================================================
// Residual block
// ==============================================================================================
namespace {

struct ResblockArgs {
  const bf16_t* x;
  bf16_t* y;
  int T, H, W;
  const wvd_resblock_weights* w;
  float eps;
  const bf16_t* hist1;
  int th1;
  const bf16_t* hist2;
  int th2;
  // workspace
  bf16_t* a;   // activated input, max(cin, cout) channels
  bf16_t* h;   // conv1 output
  bf16_t* sc;  // shortcut output (cin != cout)
};

// y = conv2(a2) + (x or shortcut(x)); a1 = SiLU(norm1(x)), h = conv1(a1), a2 = SiLU(norm2(h)).
// `after_conv1` / `after_conv2` run right after each conv (the cache updates read a1 / a2).
template <class F1, class F2>
wvd_status resblock_core(const ResblockArgs& r, hipStream_t s, F1 after_conv1, F2 after_conv2) {
  const wvd_resblock_weights* w = r.w;
  const int64_t P = (int64_t)r.T * r.H * r.W;
  const bf16_t* residual = r.x;
  if (norm_sc_fused(w->cin, w->cout, w->shortcut, w->shortcut_bias, w->gamma1)) {
    WVD_TRY(run_norm_sc(r.x, w->gamma1, r.eps, r.a, w->shortcut, w->cout, w->shortcut_bias, r.sc, P, w->cin, s));
    residual = r.sc;
  } else {
    if (w->cin != w->cout) {
      ConvProblem sc = plain_problem(r.x, nullptr, r.T, r.H, r.W, w->cin, 0, w->shortcut, w->cout, 1, 1, 1,
                                     w->shortcut_bias, r.sc, nullptr);
      WVD_TRY(run_conv(sc, s, conv_flops(P, w->cout, w->cin)));
      residual = r.sc;
    }
    WVD_TRY(run_norm(r.x, w->gamma1, r.eps, 1, r.a, P, w->cin, s));
  }
  ConvProblem c1 = plain_problem(r.a, r.hist1, r.T, r.H, r.W, w->cin, r.th1, w->conv1, w->cout, 3, 3, 3, w->bias1, r.h,
                                 nullptr);
  // conv2's input a2 = SiLU(norm2(h)): fused into conv1's epilogue when one workgroup holds every
  // output channel of a position (then h is never stored), else a separate pass
  const bool fuse = conv_can_fuse_norm(w->cout, w->bias1, w->gamma2);
  if (fuse) {
    c1.norm_gamma = w->gamma2;
    c1.norm_eps = r.eps;
    c1.norm_silu = 1;
  }
  WVD_TRY(run_conv(c1, s, conv_flops(P, w->cout, 27LL * w->cin)));
  WVD_TRY(after_conv1(r.a));
  const bf16_t* a2 = r.h;
  if (!fuse) {
    WVD_TRY(run_norm(r.h, w->gamma2, r.eps, 1, r.a, P, w->cout, s));
    a2 = r.a;
  }
  ConvProblem c2 = plain_problem(a2, r.hist2, r.T, r.H, r.W, w->cout, r.th2, w->conv2, w->cout, 3, 3, 3, w->bias2,
                                 r.y, residual);
  WVD_TRY(run_conv(c2, s, conv_flops(P, w->cout, 27LL * w->cout)));
  WVD_TRY(after_conv2(a2));
  return WVD_OK;
}

size_t resblock_ws(int cin, int cout, int64_t positions) {
  const int64_t cmax = std::max(cin, cout);
  size_t b = (size_t)round_up(positions * cmax * 2, 256) + (size_t)round_up(positions * cout * 2, 256);
  if (cin != cout) b += (size_t)round_up(positions * cout * 2, 256);
  return b;
}

wvd_status check_resblock_weights(const wvd_resblock_weights* w) {
  if (!w) return fail(WVD_ERR_ARG, "resblock weights are null");
  if (w->cin <= 0 || w->cout <= 0 || w->cin % 8 || w->cout % 8 || w->cin > 512 || w->cout > 512)
    return fail(WVD_ERR_UNSUPPORTED, "resblock channels must be multiples of 8 up to 512");
  if (!w->gamma1 || !w->conv1 || !w->gamma2 || !w->conv2) return fail(WVD_ERR_ARG, "resblock weight pointer is null");
  if (!aligned16(w->gamma1) || !aligned16(w->gamma2)) return fail(WVD_ERR_ALIGN, "gammas must be 16-byte aligned");
  if (w->cin != w->cout && !w->shortcut) return fail(WVD_ERR_ARG, "cin != cout needs the shortcut weight");
  if (!aligned16(w->conv1) || !aligned16(w->conv2) || (w->shortcut && !aligned16(w->shortcut)))
    return fail(WVD_ERR_ALIGN, "packed weights must be 16-byte aligned");
  return WVD_OK;
}

}  // namespace

extern "C" size_t wvd_resblock_workspace_bytes(int cin, int cout, int t, int h, int w) {
  if (cin <= 0 || cout <= 0 || t < 0 || h <= 0 || w <= 0) return 0;
  return resblock_ws(cin, cout, (int64_t)t * h * w);
}

extern "C" wvd_status wvd_resblock(const wvd_tensor* x, const wvd_resblock_weights* wts, float eps,
                                   const wvd_tensor* hist1, const wvd_tensor* hist2, wvd_tensor* y,
                                   wvd_tensor* hist1_out, wvd_tensor* hist2_out, void* ws, size_t ws_bytes,
                                   wvd_stream stream) {
  WVD_TRY(check_resblock_weights(wts));
  WVD_TRY(check_tensor(x, "x", WVD_BF16, WVD_NTHWC, true));
  WVD_TRY(check_tensor(y, "y", WVD_BF16, WVD_NTHWC, true));
  if (x->c != wts->cin || y->c != wts->cout || y->t != x->t || !same_grid(x, y))
    return fail(WVD_ERR_SHAPE, "x must be [1, cin, T, H, W] and y [1, cout, T, H, W]");
  if (x->data == y->data && numel(x) > 0) return fail(WVD_ERR_ARG, "y may not alias x");
  const wvd_tensor* hs[2] = {hist1, hist2};
  const wvd_tensor* ho[2] = {hist1_out, hist2_out};
  const int hc[2] = {wts->cin, wts->cout};
  int th[2] = {0, 0};
  for (int i = 0; i < 2; ++i) {
    if (hs[i]) {
      WVD_TRY(check_tensor(hs[i], i ? "hist2" : "hist1", WVD_BF16, WVD_NTHWC, true));
      if (hs[i]->c != hc[i] || !same_grid(hs[i], x) || hs[i]->t > 2)
        return fail(WVD_ERR_SHAPE, "hist%d must be [1, %d, <=2, H, W]", i + 1, hc[i]);
      th[i] = (int)hs[i]->t;
    }
  }
  for (int i = 0; i < 2; ++i) {
    if (ho[i]) {
      WVD_TRY(check_tensor(ho[i], i ? "hist2_out" : "hist1_out", WVD_BF16, WVD_NTHWC, true));
      const int want = history_frames_after((int)x->t, th[i]);
      if (ho[i]->c != hc[i] || !same_grid(ho[i], x) || ho[i]->t != want)
        return fail(WVD_ERR_SHAPE, "hist%d_out must be [1, %d, %d, H, W]", i + 1, hc[i], want);
      if (hs[i] && hs[i]->data == ho[i]->data && want > 0) return fail(WVD_ERR_ARG, "hist_out may not alias hist");
    }
  }
  if (!(eps >= 0.0f)) return fail(WVD_ERR_ARG, "eps must be >= 0");
  const int64_t P = x->t * x->h * x->w;
  const size_t need = resblock_ws(wts->cin, wts->cout, P);
  if (ws_bytes < need) return fail(WVD_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, need);
  if (P > 0 && (!ws || !aligned16(ws))) return fail(WVD_ERR_ALIGN, "workspace null or not 16-byte aligned");
  if (x->t == 0) {
    hipStream_t s = (hipStream_t)stream;
    for (int i = 0; i < 2; ++i)
      if (ho[i] && hs[i] && th[i] > 0)
        WVD_HIP(hipMemcpyAsync(ho[i]->data, hs[i]->data, (size_t)numel(hs[i]) * 2, hipMemcpyDeviceToDevice, s),
                "history copy");
    return WVD_OK;
  }
  ResblockArgs r;
  r.x = (const bf16_t*)x->data;
  r.y = (bf16_t*)y->data;
  r.T = (int)x->t;
  r.H = (int)x->h;
  r.W = (int)x->w;
  r.w = wts;
  r.eps = eps;
  r.hist1 = hist1 ? (const bf16_t*)hist1->data : nullptr;
  r.th1 = th[0];
  r.hist2 = hist2 ? (const bf16_t*)hist2->data : nullptr;
  r.th2 = th[1];
  char* base = (char*)ws;
  r.a = (bf16_t*)base;
  base += round_up(P * std::max(wts->cin, wts->cout) * 2, 256);
  r.h = (bf16_t*)base;
  base += round_up(P * wts->cout * 2, 256);
  r.sc = (bf16_t*)base;
  hipStream_t s = (hipStream_t)stream;
  const size_t fb1 = (size_t)x->h * x->w * wts->cin * 2, fb2 = (size_t)x->h * x->w * wts->cout * 2;
  return resblock_core(
      r, s,
      [&](const bf16_t* a1) {
        return hist1_out ? copy_history_out(a1, r.T, r.hist1, th[0], hist1_out->data, fb1, s) : WVD_OK;
      },
      [&](const bf16_t* a2) {
        return hist2_out ? copy_history_out(a2, r.T, r.hist2, th[1], hist2_out->data, fb2, s) : WVD_OK;
      });
}

// ==============================================================================================
// Residual block without a caller workspace
// ==============================================================================================
namespace {

// The residual block's workspace (activated input, conv1 output, shortcut output) for callers
// that cannot allocate: a file-scope device array, one copy per GPU, held until the process ends.
// In host code `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

wvd_status scratch_for_current_device(char** out) {
  int dev = -1;
  WVD_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(WVD_ERR_UNSUPPORTED, "device %d beyond the scratch table", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    WVD_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!ptr || !aligned16(ptr)) return fail(WVD_ERR_HIP, "scratch symbol has no usable device address");
    g_scratch_ptr[dev] = (char*)ptr;
  }
  *out = g_scratch_ptr[dev];
  return WVD_OK;
}

}  // namespace

extern "C" size_t wvd_resblock_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

extern "C" wvd_status wvd_resblock_noalloc(const wvd_tensor* x, const wvd_resblock_weights* wts, float eps,
                                           const wvd_tensor* hist1, const wvd_tensor* hist2, wvd_tensor* y,
                                           wvd_tensor* hist1_out, wvd_tensor* hist2_out, wvd_stream stream) {
  WVD_TRY(check_resblock_weights(wts));
  WVD_TRY(check_tensor(x, "x", WVD_BF16, WVD_NTHWC, true));
  const size_t need = resblock_ws(wts->cin, wts->cout, x->t * x->h * x->w);
  if (need > kNoAllocScratchBytes)
    return fail(WVD_ERR_WORKSPACE,
                "resblock_noalloc: this input needs %zu bytes of workspace, the built-in scratch holds %zu "
                "(use wvd_resblock with a caller workspace)",
                need, kNoAllocScratchBytes);
  char* ws = nullptr;
  WVD_TRY(scratch_for_current_device(&ws));
  return wvd_resblock(x, wts, eps, hist1, hist2, y, hist1_out, hist2_out, ws, kNoAllocScratchBytes, stream);
}

// ==============================================================================================
// Upsampling
// ==============================================================================================
extern "C" size_t wvd_upsample_workspace_bytes(int c, int t, int h, int w, int spatial, int temporal, int order) {
  if (c <= 0 || t < 0 || h <= 0 || w <= 0) return 0;
  if (spatial && temporal) {
    // the intermediate of the first step
    const int64_t inter = (order == WVD_SPATIAL_FIRST) ? (int64_t)t * 4 * h * w * c : (int64_t)2 * t * h * w * c;
    return (size_t)round_up(inter * 2, 256);
  }
  return 0;
}

extern "C" wvd_status wvd_upsample(const wvd_tensor* x, const void* spatial, const float* spatial_bias,
                                   const void* temporal, const float* temporal_bias, int order, int first,
                                   const wvd_tensor* time_hist, wvd_tensor* y, wvd_tensor* time_hist_out, void* ws,
                                   size_t ws_bytes, wvd_stream stream) {
  WVD_TRY(check_tensor(x, "x", WVD_BF16, WVD_NTHWC, true));
  WVD_TRY(check_tensor(y, "y", WVD_BF16, WVD_NTHWC, true));
  if (!spatial && !temporal) return fail(WVD_ERR_ARG, "neither step is on");
  if (order != WVD_TIME_FIRST && order != WVD_SPATIAL_FIRST) return fail(WVD_ERR_ARG, "unknown order");
  if ((spatial && !aligned16(spatial)) || (temporal && !aligned16(temporal)))
    return fail(WVD_ERR_ALIGN, "packed weights must be 16-byte aligned");
  const int C = (int)x->c, T = (int)x->t;
  if (C % 8 != 0) return fail(WVD_ERR_UNSUPPORTED, "channels must be a multiple of 8");
  const int tf = (temporal && first) ? 1 : 0;  // frames that pass through the time step
  const int64_t To = temporal ? (first ? (T > 0 ? 2LL * T - 1 : 0) : 2LL * T) : T;
  const int64_t Ho = spatial ? 2 * x->h : x->h, Wo = spatial ? 2 * x->w : x->w;
  if (y->c != C || y->t != To || y->h != Ho || y->w != Wo)
    return fail(WVD_ERR_SHAPE, "y must be [1, %d, %lld, %lld, %lld]", C, (long long)To, (long long)Ho, (long long)Wo);
  if (x->data == y->data && numel(x) > 0) return fail(WVD_ERR_ARG, "y may not alias x");
  // geometry of the time conv's input grid
  const int th_h = (int)((temporal && order == WVD_SPATIAL_FIRST && spatial) ? Ho : x->h);
  const int th_w = (int)((temporal && order == WVD_SPATIAL_FIRST && spatial) ? Wo : x->w);
  const int Tc = T - tf;  // frames the time conv sees
  int Th = 0;
  if (time_hist) {
    if (!temporal) return fail(WVD_ERR_ARG, "time_hist without a time step");
    WVD_TRY(check_tensor(time_hist, "time_hist", WVD_BF16, WVD_NTHWC, true));
    if (time_hist->c != C || time_hist->h != th_h || time_hist->w != th_w || time_hist->t > 2)
      return fail(WVD_ERR_SHAPE, "time_hist must be [1, C, <=2, h, w] of the time conv's input");
    if (first && time_hist->t > 0) return fail(WVD_ERR_STATE, "the first chunk has no time history");
    Th = (int)time_hist->t;
  }
  if (time_hist_out) {
    if (!temporal) return fail(WVD_ERR_ARG, "time_hist_out without a time step");
    WVD_TRY(check_tensor(time_hist_out, "time_hist_out", WVD_BF16, WVD_NTHWC, true));
    const int want = history_frames_after(Tc < 0 ? 0 : Tc, Th);
    if (time_hist_out->c != C || time_hist_out->h != th_h || time_hist_out->w != th_w || time_hist_out->t != want)
      return fail(WVD_ERR_SHAPE, "time_hist_out must be [1, C, %d, h, w]", want);
    if (time_hist && time_hist->data == time_hist_out->data && want > 0)
      return fail(WVD_ERR_ARG, "time_hist_out may not alias time_hist");
  }
  const size_t need = wvd_upsample_workspace_bytes(C, T, (int)x->h, (int)x->w, spatial != nullptr, temporal != nullptr, order);
  if (ws_bytes < need) return fail(WVD_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, need);
  if (need > 0 && (!ws || !aligned16(ws))) return fail(WVD_ERR_ALIGN, "workspace null or not 16-byte aligned");
  if (T == 0) {  // no frames: the time conv's history passes through unchanged
    if (time_hist_out && Th > 0)
      WVD_HIP(hipMemcpyAsync(time_hist_out->data, time_hist->data, (size_t)numel(time_hist) * 2, hipMemcpyDeviceToDevice,
                             (hipStream_t)stream),
              "history copy");
    return WVD_OK;
  }
  hipStream_t s = (hipStream_t)stream;
  const int H = (int)x->h, W = (int)x->w;
  const bf16_t* hist = time_hist ? (const bf16_t*)time_hist->data : nullptr;

  // time step: src [T][h][w][C] -> dst [To_t][h][w][C]
  auto time_step = [&](const bf16_t* src, int h, int w, bf16_t* dst) -> wvd_status {
    const size_t fb = (size_t)h * w * C * 2;
    const int To_t = first ? 2 * T - 1 : 2 * T;
    if (tf) WVD_HIP(hipMemcpyAsync(dst, src, fb, hipMemcpyDeviceToDevice, s), "first frame copy");
    if (Tc > 0) WVD_TRY(run_time_conv(src + (size_t)tf * h * w * C, hist, Tc, h, w, C, Th, temporal, temporal_bias, dst, To_t, tf, s));
    if (time_hist_out) WVD_TRY(copy_history_out(src + (size_t)tf * h * w * C, Tc, hist, Th, time_hist_out->data, fb, s));
    return WVD_OK;
  };
  if (spatial && temporal) {
    bf16_t* inter = (bf16_t*)ws;
    if (order == WVD_TIME_FIRST) {
      WVD_TRY(time_step((const bf16_t*)x->data, H, W, inter));
      WVD_TRY(run_phase_conv(inter, (int)To, H, W, C, spatial, spatial_bias, (bf16_t*)y->data, s));
    } else {
      WVD_TRY(run_phase_conv((const bf16_t*)x->data, T, H, W, C, spatial, spatial_bias, inter, s));
      WVD_TRY(time_step(inter, 2 * H, 2 * W, (bf16_t*)y->data));
    }
  } else if (spatial) {
    WVD_TRY(run_phase_conv((const bf16_t*)x->data, T, H, W, C, spatial, spatial_bias, (bf16_t*)y->data, s));
  } else {
    WVD_TRY(time_step((const bf16_t*)x->data, H, W, (bf16_t*)y->data));
  }
  return WVD_OK;
}

// ==============================================================================================
// Decoder: parameters, packing, cache, chunk driver
// ==============================================================================================
namespace {

enum ParamKind { K_CONV3 = 0, K_CONV1 = 1, K_TIME = 2, K_SPATIAL = 3, K_GAMMA = 4, K_BIAS = 5, K_HEAD = 6 };

struct Param {
  std::string name;
  int kind;
  int co, ci;          // convs; gamma/bias: co = length
  size_t offset;       // in the packed blob
  size_t bytes;
};

struct ResPlan {
  int cin, cout;
  int gamma1, w1, b1, gamma2, w2, b2, ws, bs;  // param indices (ws/bs -1 without shortcut)
  int slot1, slot2;
};

struct StagePlan {
  std::vector<ResPlan> res;
  int cin, c;    // input and output channels
  int level;     // spatial x2 steps before the stage (its resolution)
  int temporal;
  int spatial;   // ends with nearest x2 + 3x3
  int dup;       // + DupUp3D of the stage's input
  int tw, tb, time_slot;  // time conv params and cache slot (-1 if none)
  int sw, sb;             // spatial conv params (-1 if none)
};

struct Slot {
  int level, c;
  size_t offset, frame_bytes;
  size_t alloc;  // bytes in the cache: two halves of two frames, or (the fused tail's carry) two frames
};

struct Plan {
  std::vector<Param> params;
  int pq_w, pq_b;  // post_quant_conv (-1 if none)
  int conv_in_w, conv_in_b, conv_in_slot;
  std::vector<ResPlan> mid;
  int attn_gamma, attn_qkv_w, attn_qkv_b, attn_proj_w, attn_proj_b;  // mid attention (-1 if none)
  std::vector<StagePlan> stages;
  int levels;      // spatial x2 steps in all: the head's level
  int head_plain;  // conv_out as a plain 3x3x3 conv, then unpatchify (+ clamp) into the video
  int norm_out, out_w, out_b, out_slot;
  int tail_kernel;  // the fused tail kernel runs the last upsample and the head (out_slot: its carry)
  int head_carry;   // the input-stationary head (out_slot: its carried partial Z sums, two halves)
  std::vector<Slot> slots;
  size_t packed_bytes, cache_bytes;
};

// Video colours and patch: out_channels = colours * patch^2 with unpatchify (patch >= 2).
int desc_patch(const wvd_decoder_desc* d) { return d->patch >= 2 ? d->patch : 1; }
int desc_colours(const wvd_decoder_desc* d) { return d->out_channels / (desc_patch(d) * desc_patch(d)); }
int desc_levels(const wvd_decoder_desc* d) {
  int l = 0;
  for (int s = 0; s < d->n_stages; ++s) l += d->stage_no_spatial[s] ? 0 : 1;
  return l;
}

std::atomic<int> g_fuse_head{0};  // wvd_decode_fuse_head (off: measured slower, see wvd.h)

// Whether the decode runs the fused tail kernel: the last stage is a spatial x2 upsample whose
// epilogue can apply norm_out + SiLU (no time step, no DupUp3D), at 65-96 channels, and the head
// is conv_out to at most 3 colours (no unpatchify or clamp). Its output head then never reads an
// activated tensor: the head's temporal taps are carried between passes as partial sums.
bool tail_kernel_used(const wvd_decoder_desc* d) {
  const int L = d->n_stages;
  if (L < 1 || !g_fuse_head.load() || d->patch >= 2 || d->clamp) return false;
  const int c = d->stage_channels[L - 1];
  return !d->stage_no_spatial[L - 1] && !d->stage_dup[L - 1] && !d->stage_temporal[L - 1] &&
         tail_kernel_supported(c, (int)round_up(c, 32), d->out_channels);
}

wvd_status check_desc(const wvd_decoder_desc* d) {
  if (!d) return fail(WVD_ERR_ARG, "decoder desc is null");
  if (d->n_stages < 0 || d->n_stages > WVD_MAX_STAGES) return fail(WVD_ERR_ARG, "n_stages out of range");
  auto okc = [](int c) { return c > 0 && c % 8 == 0 && c <= 2048; };
  if (!okc(d->z_channels) || !okc(d->base_channels))
    return fail(WVD_ERR_UNSUPPORTED, "z and base channels must be multiples of 8 up to 2048");
  for (int s = 0; s < d->n_stages; ++s)
    if (!okc(d->stage_channels[s])) return fail(WVD_ERR_UNSUPPORTED, "stage channels must be multiples of 8 up to 2048");
  if (d->mid_resblocks < 0 || d->stage_resblocks < 0 || d->mid_resblocks > 16 || d->stage_resblocks > 16)
    return fail(WVD_ERR_ARG, "resblock counts out of range");
  if (d->patch < 0 || d->patch > 4) return fail(WVD_ERR_UNSUPPORTED, "patch must be 0..4");
  if (d->patch >= 2 ? (d->out_channels % (d->patch * d->patch) != 0 || desc_colours(d) > 4)
                    : (d->out_channels <= 0 || d->out_channels > 4))
    return fail(WVD_ERR_UNSUPPORTED, "out_channels must be 1..4 colours times patch^2");
  for (int s = 0; s < d->n_stages; ++s) {
    const int cin = s ? d->stage_channels[s - 1] : d->base_channels, co = d->stage_channels[s];
    const int ft = d->stage_temporal[s] ? 2 : 1;
    if (d->stage_no_spatial[s] && (d->stage_temporal[s] || d->stage_dup[s]))
      return fail(WVD_ERR_UNSUPPORTED, "a stage without the spatial step can have no time step or DupUp3D");
    if (d->stage_dup[s] && (co * ft * 4) % cin != 0)
      return fail(WVD_ERR_UNSUPPORTED, "DupUp3D needs out * ft * 4 to be a multiple of the stage's input channels");
  }
  if (d->mid_attention) {
    const int64_t hw = (int64_t)d->latent_h * d->latent_w;
    if (d->mid_resblocks < 1) return fail(WVD_ERR_UNSUPPORTED, "mid attention follows the first mid block");
    if (d->base_channels % 32 != 0 || hw % 8 != 0 || hw > 65536)
      return fail(WVD_ERR_UNSUPPORTED, "mid attention needs base channels % 32 == 0 and latent h*w % 8 == 0, <= 65536");
  }
  if (d->latent_h <= 0 || d->latent_w <= 0 || d->latent_h > 4096 || d->latent_w > 4096)
    return fail(WVD_ERR_ARG, "latent size out of range");
  if (!(d->eps >= 0.0f)) return fail(WVD_ERR_ARG, "eps must be >= 0");
  return WVD_OK;
}

int add_param(Plan& p, const std::string& name, int kind, int co, int ci) {
  Param q;
  q.name = name;
  q.kind = kind;
  q.co = co;
  q.ci = ci;
  switch (kind) {
    case K_CONV3: q.bytes = (size_t)packed_elems(co, ci, 27, 1) * 2; break;
    case K_CONV1: q.bytes = (size_t)packed_elems(co, ci, 1, 1) * 2; break;
    case K_TIME: q.bytes = (size_t)packed_elems(co, ci, 3, 1) * 2; break;
    case K_SPATIAL: q.bytes = (size_t)packed_elems(co, ci, 4, 4) * 2; break;
    case K_HEAD: q.bytes = (size_t)packed_elems(36, ci, 3, 1) * 2; break;
    default: q.bytes = (size_t)co * 4; break;
  }
  q.offset = 0;
  p.params.push_back(q);
  return (int)p.params.size() - 1;
}

int add_slot(Plan& p, const wvd_decoder_desc* d, int level, int c) {
  Slot s;
  s.level = level;
  s.c = c;
  s.frame_bytes = (size_t)(d->latent_h << level) * (size_t)(d->latent_w << level) * c * 2;
  s.alloc = 4 * s.frame_bytes;
  s.offset = 0;
  p.slots.push_back(s);
  return (int)p.slots.size() - 1;
}

ResPlan add_res(Plan& p, const wvd_decoder_desc* d, const std::string& pre, int cin, int cout, int level) {
  ResPlan r;
  r.cin = cin;
  r.cout = cout;
  r.gamma1 = add_param(p, pre + ".norm1.gamma", K_GAMMA, cin, 0);
  r.w1 = add_param(p, pre + ".conv1.weight", K_CONV3, cout, cin);
  r.b1 = add_param(p, pre + ".conv1.bias", K_BIAS, cout, 0);
  r.gamma2 = add_param(p, pre + ".norm2.gamma", K_GAMMA, cout, 0);
  r.w2 = add_param(p, pre + ".conv2.weight", K_CONV3, cout, cout);
  r.b2 = add_param(p, pre + ".conv2.bias", K_BIAS, cout, 0);
  r.ws = r.bs = -1;
  if (cin != cout) {
    r.ws = add_param(p, pre + ".shortcut.weight", K_CONV1, cout, cin);
    r.bs = add_param(p, pre + ".shortcut.bias", K_BIAS, cout, 0);
  }
  r.slot1 = add_slot(p, d, level, cin);
  r.slot2 = add_slot(p, d, level, cout);
  return r;
}

Plan make_plan(const wvd_decoder_desc* d) {
  Plan p;
  int c = d->base_channels;
  const int z = d->z_channels;
  p.pq_w = p.pq_b = -1;
  if (d->post_quant) {
    p.pq_w = add_param(p, "post_quant.weight", K_CONV1, z, z);
    p.pq_b = add_param(p, "post_quant.bias", K_BIAS, z, 0);
  }
  p.conv_in_w = add_param(p, "conv_in.weight", K_CONV3, c, z);
  p.conv_in_b = add_param(p, "conv_in.bias", K_BIAS, c, 0);
  p.conv_in_slot = add_slot(p, d, 0, z);
  p.attn_gamma = p.attn_qkv_w = p.attn_qkv_b = p.attn_proj_w = p.attn_proj_b = -1;
  for (int i = 0; i < d->mid_resblocks; ++i) {
    p.mid.push_back(add_res(p, d, "mid." + std::to_string(i), c, c, 0));
    if (i == 0 && d->mid_attention) {
      p.attn_gamma = add_param(p, "mid.attn.norm.gamma", K_GAMMA, c, 0);
      p.attn_qkv_w = add_param(p, "mid.attn.qkv.weight", K_CONV1, 3 * c, c);
      p.attn_qkv_b = add_param(p, "mid.attn.qkv.bias", K_BIAS, 3 * c, 0);
      p.attn_proj_w = add_param(p, "mid.attn.proj.weight", K_CONV1, c, c);
      p.attn_proj_b = add_param(p, "mid.attn.proj.bias", K_BIAS, c, 0);
    }
  }
  int level = 0;
  for (int s = 0; s < d->n_stages; ++s) {
    StagePlan st;
    const int cs = d->stage_channels[s];
    st.cin = c;
    st.level = level;
    for (int j = 0; j < d->stage_resblocks; ++j)
      st.res.push_back(
          add_res(p, d, "up." + std::to_string(s) + ".res." + std::to_string(j), j == 0 ? c : cs, cs, level));
    c = cs;
    st.c = c;
    st.temporal = d->stage_temporal[s] != 0;
    st.spatial = d->stage_no_spatial[s] == 0;
    st.dup = d->stage_dup[s] != 0;
    st.tw = st.tb = st.time_slot = -1;
    if (st.temporal) {
      st.tw = add_param(p, "up." + std::to_string(s) + ".time.weight", K_TIME, 2 * c, c);
      st.tb = add_param(p, "up." + std::to_string(s) + ".time.bias", K_BIAS, 2 * c, 0);
      st.time_slot = add_slot(p, d, level, c);
    }
    st.sw = st.sb = -1;
    if (st.spatial) {
      st.sw = add_param(p, "up." + std::to_string(s) + ".spatial.weight", K_SPATIAL, c, c);
      st.sb = add_param(p, "up." + std::to_string(s) + ".spatial.bias", K_BIAS, c, 0);
      ++level;
    }
    p.stages.push_back(st);
  }
  p.levels = level;
  p.head_plain = d->patch >= 2 || d->clamp;
  p.norm_out = add_param(p, "norm_out.gamma", K_GAMMA, c, 0);
  p.out_w = add_param(p, "conv_out.weight", p.head_plain ? K_CONV3 : K_HEAD, d->out_channels, c);
  p.out_b = add_param(p, "conv_out.bias", K_BIAS, d->out_channels, 0);
  p.out_slot = add_slot(p, d, p.levels, c);
  p.tail_kernel = tail_kernel_used(d) ? 1 : 0;
  if (p.tail_kernel) {
    // the head's carry: the partial sums of the next two output frames, [2][3][H][W] fp32
    Slot& s = p.slots[p.out_slot];
    s.frame_bytes = (size_t)(d->latent_h << p.levels) * (size_t)(d->latent_w << p.levels) * 3 * 4;
    s.alloc = 2 * s.frame_bytes;
  }
  p.head_carry = !p.tail_kernel && !p.head_plain && head_stream_supported((int)round_up(c, 32), d->out_channels);
  if (p.head_carry) {
    // the input-stationary head's carry: Z of the next two output frames as far as the frames
    // before them contribute ([2][7][H][W] fp32 x 4 per half), double-buffered (every tile reads
    // its neighbours' positions before they may have written theirs)
    Slot& s = p.slots[p.out_slot];
    s.frame_bytes = head_stream_carry_frame_bytes(d->latent_h << p.levels, d->latent_w << p.levels);
    s.alloc = 4 * s.frame_bytes;
  }
  size_t off = 0;
  for (auto& q : p.params) {
    q.offset = off;
    off += (size_t)round_up((int64_t)q.bytes, 256);
  }
  p.packed_bytes = off;
  off = 0;
  for (auto& s : p.slots) {
    s.offset = off;
    off += (size_t)round_up((int64_t)s.alloc, 256);
  }
  p.cache_bytes = off;
  return p;
}

void param_shape(const wvd_decoder_desc* d, const Param& q, int* ndim, int64_t shape[5]) {
  (void)d;
  for (int i = 0; i < 5; ++i) shape[i] = 0;
  switch (q.kind) {
    case K_CONV3:
    case K_HEAD: *ndim = 5; shape[0] = q.co; shape[1] = q.ci; shape[2] = shape[3] = shape[4] = 3; break;
    case K_CONV1: *ndim = 5; shape[0] = q.co; shape[1] = q.ci; shape[2] = shape[3] = shape[4] = 1; break;
    case K_TIME: *ndim = 5; shape[0] = q.co; shape[1] = q.ci; shape[2] = 3; shape[3] = shape[4] = 1; break;
    case K_SPATIAL: *ndim = 4; shape[0] = q.co; shape[1] = q.ci; shape[2] = shape[3] = 3; break;
    default: *ndim = 1; shape[0] = q.co; break;
  }
}

uint64_t desc_hash(const wvd_decoder_desc* d) {
  // FNV-1a over the descriptor's fields
  uint64_t h = 1469598103934665603ULL;
  const int v[] = {d->z_channels, d->base_channels, d->n_stages, d->mid_resblocks, d->stage_resblocks,
                   d->out_channels, d->latent_h, d->latent_w};
  auto mix = [&](uint32_t x) {
    for (int i = 0; i < 4; ++i) {
      h ^= (x >> (8 * i)) & 0xffu;
      h *= 1099511628211ULL;
    }
  };
  for (int x : v) mix((uint32_t)x);
  for (int s = 0; s < d->n_stages; ++s) {
    mix((uint32_t)d->stage_channels[s]);
    mix((uint32_t)d->stage_temporal[s]);
    mix((uint32_t)d->stage_no_spatial[s]);
    mix((uint32_t)d->stage_dup[s]);
  }
  mix((uint32_t)d->post_quant);
  mix((uint32_t)d->mid_attention);
  mix((uint32_t)d->patch);
  mix((uint32_t)d->clamp);
  uint32_t e;
  memcpy(&e, &d->eps, 4);
  mix(e);
  return h;
}

// Frames at each point of one chunk of n latent frames.
struct ChunkFrames {
  int64_t stage_in[WVD_MAX_STAGES];  // frames of the stage's resblocks
  int64_t stage_out[WVD_MAX_STAGES]; // after the stage's time conv
  int64_t video;
};

ChunkFrames chunk_frames(const wvd_decoder_desc* d, int64_t n, bool first_rule) {
  ChunkFrames f;
  int64_t t = n;
  for (int s = 0; s < d->n_stages; ++s) {
    f.stage_in[s] = t;
    if (d->stage_temporal[s]) t = (first_rule && t > 0) ? 2 * t - 1 : 2 * t;
    f.stage_out[s] = t;
  }
  f.video = t;
  return f;
}

// The head's tap planes: 9 planes of 4 fp32 channels per position (float4 = 16 bytes per
// position and plane), 8 bf16 elements' worth of bytes per plane and position.
constexpr int kHeadPlanes = 9;

// Workspace buffers of the chunk driver (elements of bf16).
struct WsLayout {
  size_t zc, x0, x1, a, h, sc, xm;  // byte offsets
  size_t zq, keep, qkv, sc32, prob, vt, ao, head;  // the real topology's parts (0 bytes otherwise)
  size_t total;
  int64_t tail_frames;  // frames per sub-pass of the fused last upsample + head (see run_tail)
};

// Whether a conv with c output channels can apply the next residual block's norm1 + SiLU in its
// epilogue and store its own (pre-norm) output too: the dual store, on one channel tile (the
// 3x3x3 convs up to 192 channels; the x2 phase convs from 97 to 192, their 192-wide tile).
std::atomic<int> g_fuse_norm1{1};  // wvd_decode_fuse_norm1

bool dual_store_width(int c, bool phase) {
  return g_fuse_norm1.load() && conv_can_fuse_norm_width(c) && (!phase || c > 96);
}

// Whether an x2 upsample of c channels with the dual store also applies the next block's 1x1
// shortcut (c -> cout) in that epilogue, in place of storing its pre-norm output (which only the
// shortcut reads): the 192-wide phase tile, 96 shortcut outputs, packed rows 16-byte aligned.
std::atomic<int> g_fuse_shortcut{1};  // wvd_decode_fuse_shortcut

bool shortcut_in_upsample(int c, int cout, const void* w, const float* b) {
  return g_fuse_shortcut.load() && c == 192 && cout == 96 && ((uintptr_t)w & 15) == 0 && ((uintptr_t)b & 15) == 0;
}

// Whether the last stage is a spatial upsample without a time step or DupUp3D whose epilogue
// applies norm_out + SiLU (one workgroup holds every channel; the packed parameters are
// 256-byte aligned): its output is then only the head's input. The decode runs that upsample
// and the head together in frame sub-passes, so the largest tensor of the decode, the last
// level's activation, never exists for a whole pass at once.
bool fused_tail(const wvd_decoder_desc* d) {
  const int L = d->n_stages;
  return !d->stage_no_spatial[L - 1] && !d->stage_dup[L - 1] && !d->stage_temporal[L - 1] &&
         conv_can_fuse_norm_width(d->stage_channels[L - 1]);
}

// The first stage after the last temporal upsample: from there on a pass's frames can be
// processed in sub-passes (no stage changes the frame count). 0 when no stage is temporal.
int split_stage(const wvd_decoder_desc* d) {
  int s = 0;
  for (int i = 0; i < d->n_stages; ++i)
    if (d->stage_temporal[i]) s = i + 1;
  return s;
}

// n latent frames per pass through conv_in, the middle blocks and the temporal stages; nh per
// sub-pass through the later stages and the head when split (nh < n and a temporal stage
// exists), with the split level's input for all n kept in its own buffer (xm).
WsLayout ws_layout(const wvd_decoder_desc* d, int64_t n, int64_t nh) {
  const int L = d->n_stages;
  const int split = (nh > 0 && nh < n && split_stage(d) > 0) ? split_stage(d) : L;
  const ChunkFrames fl = chunk_frames(d, n, false);  // the largest frame counts
  const ChunkFrames fh = split < L ? chunk_frames(d, nh, false) : fl;
  int64_t stream = 0, act = 0, hbuf = 0, scbuf = 0, xm = 0, keep = 0;
  const bool tail = fused_tail(d);
  const int64_t hw0 = (int64_t)d->latent_h * d->latent_w;
  auto hw = [&](int level) { return hw0 << (2 * level); };
  int c = d->base_channels;
  stream = std::max(stream, n * hw(0) * c);
  act = std::max(act, n * hw(0) * std::max(c, d->z_channels));
  hbuf = std::max(hbuf, n * hw(0) * c);
  int level = 0;
  for (int s = 0; s < L; ++s) {
    const ChunkFrames& f = s < split ? fl : fh;
    const int cs = d->stage_channels[s];
    const int sp = d->stage_no_spatial[s] ? 0 : 1;
    const int64_t P = f.stage_in[s] * hw(level);
    if (d->stage_dup[s]) keep = std::max(keep, P * c);
    stream = std::max(stream, P * std::max(c, cs));
    act = std::max(act, P * std::max(c, cs));
    hbuf = std::max(hbuf, P * cs);
    if (c != cs) scbuf = std::max(scbuf, P * cs);
    c = cs;
    // time conv output, then the spatial upsample output at the next level (for a fused tail:
    // the activated buffer, one sub-pass of frames at a time, sized below)
    act = std::max(act, f.stage_out[s] * hw(level) * c);
    stream = std::max(stream, f.stage_out[s] * hw(level) * c);
    if (!(tail && s == L - 1)) {
      stream = std::max(stream, f.stage_out[s] * hw(level + sp) * c);
      act = std::max(act, f.stage_out[s] * hw(level + sp) * c);
    }
    if (s + 1 == split && split < L) xm = fl.stage_out[s] * hw(level + sp) * c;
    level += sp;
  }
  // the head's input: norm_out's output for the whole pass, or a fused tail's sub-pass, as many
  // frames as fit in what the activated buffer holds anyway (at least one)
  int64_t tail_frames = fh.video;
  if (tail && tail_kernel_used(d)) {
    // the fused tail kernel: no activated tensor at all
  } else if (tail) {
    const int64_t per_frame = hw(level) * c;
    tail_frames = std::min<int64_t>(fh.video, std::max<int64_t>(1, act / per_frame));
    act = std::max(act, tail_frames * per_frame);
  } else {
    act = std::max(act, fh.video * hw(level) * c);
  }
  // the head's fp32 tap planes Z (9 planes x 4 floats = 72 bf16 per position) live in a stream
  // buffer when neither fused head kernel takes the channel count
  const bool head_plain = d->patch >= 2 || d->clamp;
  const int cip_out = (int)round_up(c, 32);
  if (!head_plain && !head_stream_supported(cip_out, d->out_channels) && !head_fused_supported(cip_out))
    stream = std::max(stream, tail_frames * hw(level) * kHeadPlanes * 8);
  WsLayout w;
  size_t off = 0;
  auto take = [&](int64_t elems) {
    const size_t o = off;
    off += (size_t)round_up(elems * 2, 256);
    return o;
  };
  w.zc = take(n * hw0 * d->z_channels);
  w.x0 = take(stream);
  w.x1 = take(stream);
  w.a = take(act);
  w.h = take(hbuf);
  w.sc = take(scbuf);
  w.xm = take(xm);
  w.zq = take(d->post_quant ? n * hw0 * d->z_channels : 0);
  w.keep = take(keep);
  const int64_t c0 = d->base_channels;
  const bool at = d->mid_attention != 0;
  w.qkv = take(at ? 3 * n * hw0 * c0 + 32 * c0 : 0);  // (+ 32 rows: the key tile's padding reads)
  w.sc32 = take(at ? 2 * hw0 * hw0 : 0);             // fp32 scores of one frame
  w.prob = take(at ? hw0 * hw0 : 0);
  w.vt = take(at ? c0 * round_up(hw0, 32) : 0);
  w.ao = take(at ? n * hw0 * c0 : 0);
  w.head = take(head_plain ? fh.video * hw(level) * d->out_channels : 0);
  w.total = off;
  w.tail_frames = tail_frames;
  return w;
}

}  // namespace

struct wvd_cache_s {
  uint64_t hash;
  int tail_kernel;  // the plan's fused-tail mode when the cache was made (it sets the head slot's layout)
  char* storage;
  std::vector<int> valid;  // frames held per slot (right-aligned)
  std::vector<int> half;   // the slot half holding them
  int64_t next_latent;
  int64_t next_frame;
  int rule;  // first_frame_rule of the decode in progress (-1 before the first chunk)
};

extern "C" int wvd_decoder_param_count(const wvd_decoder_desc* d) {
  if (check_desc(d) != WVD_OK) return -1;
  return (int)make_plan(d).params.size();
}

extern "C" wvd_status wvd_decoder_param_info(const wvd_decoder_desc* d, int index, const char** name, int* ndim,
                                             int64_t shape[5]) {
  WVD_TRY(check_desc(d));
  // names live in a per-thread table so the returned pointers stay valid after the call
  thread_local std::vector<std::string> names;
  const Plan p = make_plan(d);
  if (index < 0 || index >= (int)p.params.size()) return fail(WVD_ERR_ARG, "parameter index out of range");
  names.resize(p.params.size());
  names[index] = p.params[index].name;
  if (name) *name = names[index].c_str();
  int nd = 0;
  int64_t sh[5];
  param_shape(d, p.params[index], &nd, sh);
  if (ndim) *ndim = nd;
  if (shape)
    for (int i = 0; i < 5; ++i) shape[i] = sh[i];
  return WVD_OK;
}

extern "C" size_t wvd_decoder_packed_bytes(const wvd_decoder_desc* d) {
  if (check_desc(d) != WVD_OK) return 0;
  return make_plan(d).packed_bytes;
}

extern "C" wvd_status wvd_decoder_pack(const wvd_decoder_desc* d, const float* const* params, void* packed,
                                       wvd_stream stream) {
  WVD_TRY(check_desc(d));
  if (!params || !packed) return fail(WVD_ERR_ARG, "null params or packed buffer");
  if (!aligned16(packed)) return fail(WVD_ERR_ALIGN, "packed buffer not 16-byte aligned");
  const Plan p = make_plan(d);
  for (size_t i = 0; i < p.params.size(); ++i)
    if (!params[i]) return fail(WVD_ERR_ARG, "parameter %zu (%s) is null", i, p.params[i].name.c_str());
  hipStream_t s = (hipStream_t)stream;
  for (size_t i = 0; i < p.params.size(); ++i) {
    const Param& q = p.params[i];
    char* dst = (char*)packed + q.offset;
    const int npad = (int)round_up(q.co, 32), cip = (int)round_up(q.ci, 32);
    switch (q.kind) {
      case K_CONV3:
        WVD_HIP(launch_pack_conv(params[i], 0, q.co, q.ci, 27, npad, cip, (bf16_t*)dst, s), "pack launch");
        break;
      case K_CONV1:
        WVD_HIP(launch_pack_conv(params[i], 0, q.co, q.ci, 1, npad, cip, (bf16_t*)dst, s), "pack launch");
        break;
      case K_TIME:
        WVD_HIP(launch_pack_conv(params[i], 0, q.co, q.ci, 3, npad, cip, (bf16_t*)dst, s), "pack launch");
        break;
      case K_SPATIAL:
        WVD_HIP(launch_pack_phase2x(params[i], 0, q.co, q.ci, npad, cip, (bf16_t*)dst, s), "pack launch");
        break;
      case K_HEAD:
        WVD_HIP(launch_pack_head(params[i], 0, q.co, q.ci, (int)round_up(36, 32), cip, (bf16_t*)dst, s),
                "pack launch");
        break;
      default:
        WVD_HIP(launch_copy_f32(params[i], (float*)dst, q.co, s), "copy launch");
        break;
    }
  }
  return WVD_OK;
}

extern "C" size_t wvd_cache_bytes(const wvd_decoder_desc* d) {
  if (check_desc(d) != WVD_OK) return 0;
  return make_plan(d).cache_bytes;
}

extern "C" wvd_status wvd_cache_init(const wvd_decoder_desc* d, void* storage, wvd_cache* out) {
  WVD_TRY(check_desc(d));
  if (!out) return fail(WVD_ERR_ARG, "out is null");
  if (!storage || !aligned16(storage)) return fail(WVD_ERR_ALIGN, "cache storage null or not 16-byte aligned");
  const Plan p = make_plan(d);
  wvd_cache c = new (std::nothrow) wvd_cache_s;
  if (!c) return fail(WVD_ERR_ARG, "out of host memory");
  c->hash = desc_hash(d);
  c->tail_kernel = p.tail_kernel;
  c->storage = (char*)storage;
  c->valid.assign(p.slots.size(), 0);
  c->half.assign(p.slots.size(), 0);
  c->next_latent = 0;
  c->next_frame = 0;
  c->rule = -1;
  *out = c;
  return WVD_OK;
}

extern "C" wvd_status wvd_cache_reset(wvd_cache c) {
  if (!c) return fail(WVD_ERR_ARG, "cache is null");
  std::fill(c->valid.begin(), c->valid.end(), 0);
  std::fill(c->half.begin(), c->half.end(), 0);
  c->next_latent = 0;
  c->next_frame = 0;
  c->rule = -1;
  return WVD_OK;
}

extern "C" void wvd_cache_destroy(wvd_cache c) { delete c; }
extern "C" int64_t wvd_cache_next_latent(wvd_cache c) { return c ? c->next_latent : -1; }

extern "C" size_t wvd_decode_workspace_bytes(const wvd_decoder_desc* d, int max_latent_frames) {
  if (check_desc(d) != WVD_OK || max_latent_frames <= 0) return 0;
  return ws_layout(d, max_latent_frames, max_latent_frames).total;
}

extern "C" size_t wvd_decode_workspace_bytes_split(const wvd_decoder_desc* d, int max_latent_frames,
                                                   int high_latent_frames) {
  if (check_desc(d) != WVD_OK || max_latent_frames <= 0 || high_latent_frames < 0) return 0;
  return ws_layout(d, max_latent_frames, high_latent_frames).total;
}

extern "C" int64_t wvd_chunk_video_frames(const wvd_decoder_desc* d, int64_t n, int first, int first_frame_rule) {
  if (check_desc(d) != WVD_OK || n < 0) return -1;
  return chunk_frames(d, n, first && first_frame_rule).video;
}

namespace {

// One chunk of n latent frames. With 0 < nh < n the stages after the last temporal upsample
// and the head run in sub-passes of nh latent frames (the first one holding the chunk's first
// latent frame), each with the caches the previous one left: the same operands in the same
// order as one pass, so the same bits, while the early stages see all n frames at once.
wvd_status decode_chunk_impl(const wvd_decoder_desc* d, const void* packed, wvd_cache cache, const wvd_tensor* z,
                             int first, int first_frame_rule, wvd_tensor* video, int64_t frame_offset, int64_t nh,
                             void* ws, size_t ws_bytes, wvd_stream stream) {
  WVD_TRY(check_desc(d));
  if (!packed || !aligned16(packed)) return fail(WVD_ERR_ALIGN, "packed weights null or not 16-byte aligned");
  if (!cache) return fail(WVD_ERR_ARG, "cache is null");
  if (cache->hash != desc_hash(d)) return fail(WVD_ERR_STATE, "the cache belongs to another decoder");
  WVD_TRY(check_tensor(z, "z", WVD_BF16, -1, false));
  WVD_TRY(check_tensor(video, "video", WVD_BF16, WVD_NCTHW, true));
  if (z->c != d->z_channels || z->h != d->latent_h || z->w != d->latent_w)
    return fail(WVD_ERR_SHAPE, "z must be [1, %d, n, %d, %d]", d->z_channels, d->latent_h, d->latent_w);
  if ((first != 0) != (cache->next_latent == 0))
    return fail(WVD_ERR_STATE, first ? "first chunk on a cache that has history (reset it)"
                                     : "not the first chunk, but the cache is empty");
  if (!first && cache->rule != (first_frame_rule != 0))
    return fail(WVD_ERR_STATE, "first_frame_rule changed within a decode");
  if (frame_offset != cache->next_frame)
    return fail(WVD_ERR_STATE, "frame_offset %lld, the previous chunk ended at %lld", (long long)frame_offset,
                (long long)cache->next_frame);
  if (nh < 0) return fail(WVD_ERR_ARG, "negative sub-pass size");
  const int64_t n = z->t;
  const bool rule = first && first_frame_rule;
  const ChunkFrames fr = chunk_frames(d, n, rule);
  const int L = d->n_stages;
  const int colours = desc_colours(d), patch = desc_patch(d);
  const int64_t vh = ((int64_t)d->latent_h << desc_levels(d)) * patch;
  const int64_t vw = ((int64_t)d->latent_w << desc_levels(d)) * patch;
  if (video->c != colours || video->h != vh || video->w != vw)
    return fail(WVD_ERR_SHAPE, "video must be [1, %d, F, %lld, %lld]", colours, (long long)vh, (long long)vw);
  if (frame_offset < 0 || frame_offset + fr.video > video->t)
    return fail(WVD_ERR_SHAPE, "chunk frames %lld..%lld do not fit a video of %lld frames", (long long)frame_offset,
                (long long)(frame_offset + fr.video), (long long)video->t);
  if (n > 4096) return fail(WVD_ERR_UNSUPPORTED, "chunk too long");
  const int split = (nh > 0 && nh < n && split_stage(d) > 0) ? split_stage(d) : L;
  const WsLayout wl = ws_layout(d, n, split < L ? nh : n);
  if (ws_bytes < wl.total) return fail(WVD_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, wl.total);
  if (!ws || !aligned16(ws)) return fail(WVD_ERR_ALIGN, "workspace null or not 16-byte aligned");

  hipStream_t s = (hipStream_t)stream;
  const Plan p = make_plan(d);
  if (cache->tail_kernel != p.tail_kernel)
    return fail(WVD_ERR_STATE, "the cache was made with the fused head %s (wvd_decode_fuse_head)",
                cache->tail_kernel ? "on" : "off");
  const char* pk = (const char*)packed;
  auto W_ = [&](int idx) -> const void* { return pk + p.params[idx].offset; };
  auto F_ = [&](int idx) -> const float* { return (const float*)(pk + p.params[idx].offset); };
  char* wsb = (char*)ws;
  bf16_t* zc = (bf16_t*)(wsb + wl.zc);
  bf16_t* bx[2] = {(bf16_t*)(wsb + wl.x0), (bf16_t*)(wsb + wl.x1)};
  bf16_t* ba = (bf16_t*)(wsb + wl.a);
  bf16_t* bh = (bf16_t*)(wsb + wl.h);
  bf16_t* bsc = (bf16_t*)(wsb + wl.sc);
  bf16_t* bxm = (bf16_t*)(wsb + wl.xm);
  bf16_t* bzq = (bf16_t*)(wsb + wl.zq);
  bf16_t* bkeep = (bf16_t*)(wsb + wl.keep);
  bf16_t* bqkv = (bf16_t*)(wsb + wl.qkv);
  float* bs32 = (float*)(wsb + wl.sc32);
  bf16_t* bprob = (bf16_t*)(wsb + wl.prob);
  bf16_t* bvt = (bf16_t*)(wsb + wl.vt);
  bf16_t* bao = (bf16_t*)(wsb + wl.ao);
  bf16_t* bhead = (bf16_t*)(wsb + wl.head);
  auto slot_ptr = [&](int slot) { return (bf16_t*)(cache->storage + p.slots[slot].offset); };
  auto slot_hist = [&](int slot) -> const bf16_t* {
    const int v = cache->valid[slot];
    const size_t fb = p.slots[slot].frame_bytes;
    return v ? (const bf16_t*)((char*)slot_ptr(slot) + (size_t)cache->half[slot] * 2 * fb + (2 - v) * fb) : nullptr;
  };
  // conv with the slot's history; the slot update from the conv's input is its side work
  auto cached_conv = [&](ConvProblem cp, int slot, const bf16_t* input, int T, double flops) -> wvd_status {
    cp.hist = slot_hist(slot);
    cp.Th = cache->valid[slot];
    int v = cache->valid[slot], h = cache->half[slot];
    slot_update_job((char*)slot_ptr(slot), h, v, input, T, p.slots[slot].frame_bytes, cp.copy);
    WVD_TRY(run_conv(cp, s, flops));
    cache->valid[slot] = v;
    cache->half[slot] = h;
    return WVD_OK;
  };

  // latents in NTHWC
  const bf16_t* zin = (const bf16_t*)z->data;
  if (z->layout == WVD_NCTHW) {
    const double zb = 4.0 * (double)d->z_channels * n * d->latent_h * d->latent_w;
    WVD_TRY(run_mem(MEM_CONVERT, zb, s, "convert launch", [&] {
      return launch_convert(z->data, 1, 1, zc, 1, 0, d->z_channels, (int)n, d->latent_h, d->latent_w, s);
    }));
    zin = zc;
  }
  if (p.pq_w >= 0) {  // post_quant_conv: 1x1x1, no history
    const int64_t P = n * d->latent_h * d->latent_w;
    ConvProblem cp = plain_problem(zin, nullptr, (int)n, d->latent_h, d->latent_w, d->z_channels, 0, W_(p.pq_w),
                                   d->z_channels, 1, 1, 1, F_(p.pq_b), bzq, nullptr);
    WVD_TRY(run_conv(cp, s, conv_flops(P, d->z_channels, d->z_channels)));
    zin = bzq;
  }
  int cur = 0;  // index of the stream buffer holding the activation
  int H = d->latent_h, Wd = d->latent_w;
  int64_t T = n;
  int c = d->base_channels;
  {
    const int64_t P = T * H * Wd;
    ConvProblem cp = plain_problem(zin, nullptr, (int)T, H, Wd, d->z_channels, 0, W_(p.conv_in_w), c, 3, 3, 3,
                                   F_(p.conv_in_b), bx[cur], nullptr);
    WVD_TRY(cached_conv(cp, p.conv_in_slot, zin, (int)T, conv_flops(P, c, 27LL * d->z_channels)));
  }
  // a residual block reading x (the stream buffer, or the split level's input) and writing the
  // stream buffer (in place when the residual is x itself). pre_act: SiLU(norm1(x)) is already in
  // the activated buffer (the producer's dual store). next_gamma: the next block's norm1 gain, when
  // conv2 also writes SiLU(norm1_next(y)) into the activated buffer (its dual store).
  // sc_ready: the shortcut's output is already in its buffer (the producer's epilogue), and x is
  // read by nothing.
  auto resblock = [&](const ResPlan& r, const bf16_t* x, bool pre_act, const float* next_gamma,
                      bool sc_ready = false) -> wvd_status {
    const int64_t P = T * H * Wd;
    bf16_t* y = bx[cur];
    const bf16_t* residual = x;
    if (sc_ready) {
      if (r.cin == r.cout || !pre_act) return fail(WVD_ERR_STATE, "a fused shortcut needs the pre-activated input");
      residual = bsc;
    } else if (!pre_act && norm_sc_fused(r.cin, r.cout, W_(r.ws), F_(r.bs), F_(r.gamma1))) {
      // norm1 and the shortcut from one read of x
      WVD_TRY(run_norm_sc(x, F_(r.gamma1), d->eps, ba, W_(r.ws), r.cout, F_(r.bs), bsc, P, r.cin, s));
      residual = bsc;
      pre_act = true;
    } else if (r.cin != r.cout) {
      ConvProblem sc = plain_problem(x, nullptr, (int)T, H, Wd, r.cin, 0, W_(r.ws), r.cout, 1, 1, 1, F_(r.bs), bsc, nullptr);
      WVD_TRY(run_conv(sc, s, conv_flops(P, r.cout, r.cin)));
      residual = bsc;
    }
    if (!pre_act) WVD_TRY(run_norm(x, F_(r.gamma1), d->eps, 1, ba, P, r.cin, s));
    ConvProblem c1 = plain_problem(ba, nullptr, (int)T, H, Wd, r.cin, 0, W_(r.w1), r.cout, 3, 3, 3, F_(r.b1), bh, nullptr);
    // norm2 + SiLU fused into conv1's epilogue when one workgroup holds all output channels
    const bool fuse = conv_can_fuse_norm(r.cout, F_(r.b1), F_(r.gamma2));
    if (fuse) {
      c1.norm_gamma = F_(r.gamma2);
      c1.norm_eps = d->eps;
      c1.norm_silu = 1;
    }
    WVD_TRY(cached_conv(c1, r.slot1, ba, (int)T, conv_flops(P, r.cout, 27LL * r.cin)));
    const bf16_t* a2 = bh;
    if (!fuse) {
      WVD_TRY(run_norm(bh, F_(r.gamma2), d->eps, 1, ba, P, r.cout, s));
      a2 = ba;
    }
    ConvProblem c2 = plain_problem(a2, nullptr, (int)T, H, Wd, r.cout, 0, W_(r.w2), r.cout, 3, 3, 3, F_(r.b2), y, residual);
    if (next_gamma) {
      // y = conv2 + bias + residual into the stream buffer, SiLU(norm1_next(y)) into the
      // activated buffer (free: conv2 reads a2 from the conv1 output, fused there at this width)
      if (a2 == ba) return fail(WVD_ERR_STATE, "dual store needs conv1's fused norm");
      c2.y_pre = y;
      c2.y = ba;
      c2.norm_gamma = next_gamma;
      c2.norm_eps = d->eps;
      c2.norm_silu = 1;
    }
    WVD_TRY(cached_conv(c2, r.slot2, a2, (int)T, conv_flops(P, r.cout, 27LL * r.cout)));
    return WVD_OK;
  };
  // the next stage's first residual block takes its SiLU(norm1(x)) from the activated buffer,
  // written by this stage's x2 upsample (its dual store)
  bool stage_pre_act = false;
  bool stage_sc_ready = false;  // the next stage's first shortcut is in bsc (the upsample's epilogue)
  bool mid_pre_act = false;
  // The mid block's attention, in place on x (level 0, T frames): n = RMS norm of x; q | k | v
  // from one 1x1 conv C -> 3C whose channel thirds go to frames t, T + t, 2T + t; per frame the
  // scores q k^T as a 1x1 conv of q whose weight rows are the frame's keys (fp32 out), the row
  // softmax of scores / sqrt(C), o = P v as a 1x1 conv of P whose weight rows are the frame's
  // values transposed; then proj + bias + x.
  auto run_attention = [&](bf16_t* x) -> wvd_status {
    const int hw = H * Wd;
    const int64_t P = T * hw;
    const int ldk = (int)round_up(hw, 32);
    WVD_TRY(run_norm(x, F_(p.attn_gamma), d->eps, 0, ba, P, c, s));
    ConvProblem qp = plain_problem(ba, nullptr, (int)T, H, Wd, c, 0, W_(p.attn_qkv_w), 3 * c, 1, 1, 1,
                                   F_(p.attn_qkv_b), bqkv, nullptr);
    qp.nsplit = c;
    qp.fstride = (int)T;
    qp.To = 3 * (int)T;
    WVD_TRY(run_conv(qp, s, conv_flops(P, 3 * c, c)));
    for (int64_t t = 0; t < T; ++t) {
      const bf16_t* q = bqkv + (size_t)t * hw * c;
      const bf16_t* k = bqkv + (size_t)(T + t) * hw * c;
      const bf16_t* v = bqkv + (size_t)(2 * T + t) * hw * c;
      ConvProblem sp = plain_problem(q, nullptr, 1, H, Wd, c, 0, k, hw, 1, 1, 1, nullptr, nullptr, nullptr);
      sp.y = bs32;
      sp.y_f32 = 1;
      WVD_TRY(run_conv(sp, s, conv_flops(hw, hw, c)));
      WVD_TRY(run_mem(MEM_ATTN, (double)hw * hw * 14.0, s, "softmax launch", [&] {
        return launch_softmax_rows(bs32, hw, hw, hw, 1.0f / std::sqrt((float)c), bprob, hw, s);
      }));
      WVD_TRY(run_mem(MEM_ATTN, (double)hw * c * 2.0 + (double)c * ldk * 2.0, s, "transpose launch",
                      [&] { return launch_transpose_pad(v, hw, c, bvt, ldk, s); }));
      ConvProblem op = plain_problem(bprob, nullptr, 1, H, Wd, hw, 0, bvt, c, 1, 1, 1, nullptr,
                                     bao + (size_t)t * hw * c, nullptr);
      WVD_TRY(run_conv(op, s, conv_flops(hw, c, hw)));
    }
    ConvProblem pp = plain_problem(bao, nullptr, (int)T, H, Wd, c, 0, W_(p.attn_proj_w), c, 1, 1, 1,
                                   F_(p.attn_proj_b), x, x);
    return run_conv(pp, s, conv_flops(P, c, c));
  };
  for (size_t i = 0; i < p.mid.size(); ++i) {
    // (the middle blocks run at the base width; the attention sits between the first two)
    const bool dual = i + 1 < p.mid.size() && !(i == 0 && p.attn_qkv_w >= 0) &&
                      p.mid[i + 1].cin == p.mid[i].cout && dual_store_width(p.mid[i].cout, false);
    WVD_TRY(resblock(p.mid[i], bx[cur], i > 0 && mid_pre_act, dual ? F_(p.mid[i + 1].gamma1) : nullptr));
    mid_pre_act = dual;
    if (i == 0 && p.attn_qkv_w >= 0) WVD_TRY(run_attention(bx[cur]));
  }
  // The last stage's spatial upsample also applies norm_out + SiLU in its epilogue when one
  // workgroup holds every channel (the L4 tensor is then written once, already activated).
  const bf16_t* act = nullptr;  // conv_out's input once norm_out has been applied
  bf16_t* zbuf = nullptr;       // a free buffer for the head's tap planes
  // A fused tail (fused_tail): the last upsample's input, its size and stage, recorded by
  // run_stage and consumed by run_tail.
  const bool tail = fused_tail(d);
  const bf16_t* tail_x = nullptr;
  int tail_h = 0, tail_w = 0, tail_stage = -1;
  // one stage: its residual blocks (the first reading x), its time conv and spatial upsample
  // (into `up`, or the stream buffers)
  auto run_stage = [&](int si, const bf16_t* x, bf16_t* up) -> wvd_status {
    const StagePlan& st = p.stages[si];
    const int64_t T_in = T;
    const int H_in = H, W_in = Wd;
    if (st.dup && T_in > 0)  // the stage's input, for its DupUp3D shortcut after the upsampling
      WVD_HIP(hipMemcpyAsync(bkeep, x, (size_t)T_in * H_in * W_in * st.cin * 2, hipMemcpyDeviceToDevice, s),
              "DupUp3D source copy");
    bool pre_act = stage_pre_act;
    bool sc_ready = stage_sc_ready;
    stage_pre_act = false;
    stage_sc_ready = false;
    if (sc_ready && st.res.empty()) return fail(WVD_ERR_STATE, "a fused shortcut without its block");
    for (size_t k = 0; k < st.res.size(); ++k) {
      const ResPlan& r = st.res[k];
      const bool dual = k + 1 < st.res.size() && st.res[k + 1].cin == r.cout && dual_store_width(r.cout, false);
      WVD_TRY(resblock(r, x, pre_act, dual ? F_(st.res[k + 1].gamma1) : nullptr, k == 0 && sc_ready));
      pre_act = dual;
      x = bx[cur];
      c = r.cout;
    }
    if (!st.spatial) return WVD_OK;  // (no time step or DupUp3D either)
    const bool fuse_out = si == L - 1 && !st.dup && conv_can_fuse_norm(c, F_(st.sb), F_(p.norm_out));
    if (tail && si == L - 1 && !fuse_out) return fail(WVD_ERR_ALIGN, "norm_out or the last upsample's bias unaligned");
    const float* ng = fuse_out ? F_(p.norm_out) : nullptr;
    bf16_t* yout = nullptr;  // the upsampling's output
    if (st.temporal) {
      const size_t fb = (size_t)H * Wd * c * 2;
      const int tf = rule ? 1 : 0;
      const int64_t To = fr.stage_out[si];
      const int Tc = (int)(T - tf);
      bf16_t* dst = ba;  // the activated buffer is free here
      if (tf && T > 0) WVD_HIP(hipMemcpyAsync(dst, x, fb, hipMemcpyDeviceToDevice, s), "first frame copy");
      if (Tc > 0) {
        const bf16_t* src = x + (size_t)tf * H * Wd * c;
        ConvProblem cp = plain_problem(src, nullptr, Tc, H, Wd, c, 0, W_(st.tw), 2 * c, 3, 1, 1, F_(st.tb), dst, nullptr);
        cp.To = (int)To;
        cp.nsplit = c;
        cp.fmul = 2;
        cp.fbase = tf;
        WVD_TRY(cached_conv(cp, st.time_slot, src, Tc, conv_flops((int64_t)Tc * H * Wd, 2 * c, 3LL * c)));
      }
      T = To;
      // spatial upsample from the time conv's output into the stream buffer (or `up`)
      bf16_t* out = up ? up : bx[cur];
      WVD_TRY(run_phase_conv(dst, (int)T, H, Wd, c, W_(st.sw), F_(st.sb), out, s, ng, d->eps));
      yout = out;
      if (fuse_out) {
        act = out;
        zbuf = bx[cur ^ 1];
      }
    } else if (fuse_out && tail) {
      // the fused tail: this upsample runs with the head, in frame sub-passes (run_tail)
      tail_x = x;
      tail_h = H;
      tail_w = Wd;
      tail_stage = si;
    } else if (fuse_out) {
      WVD_TRY(run_phase_conv(x, (int)T, H, Wd, c, W_(st.sw), F_(st.sb), ba, s, ng, d->eps));
      act = ba;
      zbuf = bx[cur ^ 1];
    } else if (up) {
      WVD_TRY(run_phase_conv(x, (int)T, H, Wd, c, W_(st.sw), F_(st.sb), up, s));
      yout = up;
    } else {
      // the next stage's first block's norm1 + SiLU in the epilogue too (dual store), when nothing
      // is added to the upsampled output first (DupUp3D) and the widths allow it
      const bool dual = !st.dup && si + 1 < L && !p.stages[si + 1].res.empty() &&
                        p.stages[si + 1].res[0].cin == c && dual_store_width(c, true);
      const ResPlan* r0 = dual ? &p.stages[si + 1].res[0] : nullptr;
      if (dual && r0->cout != c && r0->ws >= 0 && shortcut_in_upsample(c, r0->cout, W_(r0->ws), F_(r0->bs))) {
        // the pre-norm output is read by the block's 1x1 shortcut alone: its product goes to the
        // shortcut buffer instead, and the stream buffer is not written
        WVD_TRY(run_phase_conv(x, (int)T, H, Wd, c, W_(st.sw), F_(st.sb), ba, s, F_(r0->gamma1), d->eps, nullptr,
                               W_(r0->ws), F_(r0->bs), r0->cout, bsc));
        stage_pre_act = true;
        stage_sc_ready = true;
      } else if (dual) {
        WVD_TRY(run_phase_conv(x, (int)T, H, Wd, c, W_(st.sw), F_(st.sb), ba, s, F_(p.stages[si + 1].res[0].gamma1),
                               d->eps, bx[cur ^ 1]));
        stage_pre_act = true;
      } else {
        WVD_TRY(run_phase_conv(x, (int)T, H, Wd, c, W_(st.sw), F_(st.sb), bx[cur ^ 1], s));
      }
      cur ^= 1;
      yout = bx[cur];
    }
    if (st.dup) {
      // + DupUp3D of the stage input; on the pass holding latent frame 0 that frame's first
      // time copy is dropped, as the time step passed it through once
      const int ft = st.temporal ? 2 : 1, fo = (st.temporal && rule) ? 1 : 0;
      const double db = (double)T * 4 * H_in * W_in * c * 4.0 + (double)T_in * H_in * W_in * st.cin * 2.0;
      WVD_TRY(run_mem(MEM_DUP, db, s, "DupUp3D launch", [&] {
        return launch_dup_add(yout, bkeep, (int)T, (int)T_in, H_in, W_in, st.cin, c, ft, fo, s);
      }));
    }
    H *= 2;
    Wd *= 2;
    return WVD_OK;
  };
  // norm_out + SiLU (unless fused above), then conv_out and the 9-tap stencil into the video
  // (NCTHW) at frame `fo`
  auto run_head = [&](int64_t fo) -> wvd_status {
    const int64_t P = T * H * Wd;
    if (!act) {
      WVD_TRY(run_norm(bx[cur], F_(p.norm_out), d->eps, 1, ba, P, c, s));
      act = ba;
      zbuf = bx[cur ^ 1];
    }
    if (p.head_plain) {
      // conv_out as a plain causal 3x3x3 conv to colours * patch^2 channels, then unpatchify
      // (+ clamp) into the video
      const int co = d->out_channels;
      ConvProblem cp = plain_problem(act, nullptr, (int)T, H, Wd, c, 0, W_(p.out_w), co, 3, 3, 3, F_(p.out_b), bhead,
                                     nullptr);
      WVD_TRY(cached_conv(cp, p.out_slot, act, (int)T, conv_flops(P, co, 27LL * c)));
      return run_mem(MEM_UNPATCH, (double)P * co * 4.0, s, "unpatchify launch", [&] {
        return launch_unpatchify(bhead, (int)T, H, Wd, colours, patch, d->clamp, (bf16_t*)video->data, video->t,
                                 (int)fo, s);
      });
    }
    const int co = d->out_channels;
    const int cip = (int)round_up(c, 32);
    if (head_stream_supported(cip, co) || head_fused_supported(cip)) {
      // tap conv + stencil in one kernel (no tap planes in memory); reads the activation once,
      // writes co bf16 channels; the input-stationary kernel up to 96 channels and 3 colours
      // (with the frames before it as a carry), else the frame-tiled one (with the slot's
      // history frames)
      const int slot = p.out_slot;
      if (head_stream_supported(cip, co)) {
        // the frames before this launch come in as the carried partial sums of the slot's
        // current half; the launch leaves its own in the other half
        if (!p.head_carry) return fail(WVD_ERR_STATE, "the head's cache slot holds no carry");
        if (T == 0) return WVD_OK;
        const size_t cfb = p.slots[slot].frame_bytes;
        char* sp = (char*)slot_ptr(slot);
        const float* cin = cache->valid[slot] ? (const float*)(sp + (size_t)cache->half[slot] * 2 * cfb) : nullptr;
        float* cout = (float*)(sp + (size_t)(cache->half[slot] ^ 1) * 2 * cfb);
        // reads the activation once and both carries, writes co bf16 channels
        const double hb = (double)P * c * 2.0 + (double)P * co * 2.0 + (cin ? 2.0 : 0.0) * cfb + 2.0 * cfb;
        WVD_TRY(run_mem(MEM_HEAD_STREAM, hb, s, "head launch", [&] {
          return launch_head_stream(act, (int)T, H, Wd, c, cip, (const bf16_t*)W_(p.out_w), F_(p.out_b), co,
                                    (bf16_t*)video->data, video->t, (int)fo, cin, cout, s);
        }));
        cache->half[slot] ^= 1;
        cache->valid[slot] = (int)std::min<int64_t>(2, cache->valid[slot] + T);
        return WVD_OK;
      }
      const bf16_t* hist = slot_hist(slot);
      const int Th = cache->valid[slot];
      const double hb = (double)(T + std::min(Th, 2)) * H * Wd * c * 2.0 + (double)P * co * 2.0;
      // the slot update from the activation is the head launch's side work
      int v = cache->valid[slot], h = cache->half[slot];
      CopyJob job;
      slot_update_job((char*)slot_ptr(slot), h, v, act, (int)T, p.slots[slot].frame_bytes, job);
      WVD_TRY(run_mem(MEM_HEAD_FUSED, hb, s, "head launch", [&] {
        return launch_head_fused(act, hist, Th, (int)T, H, Wd, c, cip, (const bf16_t*)W_(p.out_w), F_(p.out_b), co,
                                 (bf16_t*)video->data, video->t, (int)fo, s, &job);
      }));
      cache->valid[slot] = v;
      cache->half[slot] = h;
      return WVD_OK;
    }
    float* Z = (float*)zbuf;
    // n = tap*4 + o: each lane's 4 accumulator channels are one tap's 4 colour slots, stored as
    // one float4 into plane `tap`: frame f = t + T*tap of a [9T][H][W][4] tensor
    ConvProblem cp = plain_problem(act, nullptr, (int)T, H, Wd, c, 0, W_(p.out_w), 36, 3, 1, 1, nullptr, nullptr,
                                   nullptr);
    cp.y = Z;
    cp.y_f32 = 1;
    cp.nsplit = 4;
    cp.fstride = (int)T;
    cp.To = (int)T * kHeadPlanes;
    WVD_TRY(cached_conv(cp, p.out_slot, act, (int)T, conv_flops(P, co, 27LL * c)));
    // reads the 9 tap planes (16 bytes per plane and position), writes co bf16 channels
    const double hb = (double)P * (kHeadPlanes * 16.0 + 2.0 * co);
    return run_mem(MEM_HEAD_STENCIL, hb, s, "head launch", [&] {
      return launch_head_stencil(Z, co, F_(p.out_b), (bf16_t*)video->data, video->t, (int)fo, (int)T, H, Wd, s);
    });
  };
  // The fused tail: the last upsample (norm_out + SiLU in its epilogue) and the head in sub-passes
  // of wl.tail_frames frames, each written into the activated buffer and consumed by the head
  // (whose cache slot carries the two frames before each sub-pass); otherwise just the head.
  auto run_tail = [&](int64_t fo) -> wvd_status {
    if (!tail_x) return run_head(fo);
    const StagePlan& st = p.stages[tail_stage];
    const int64_t Tall = T;
    if (p.tail_kernel) {
      // the fused tail kernel: the x2 upsample with norm_out + SiLU and the head in one launch
      // over the pass; the head's temporal taps come in and go out as the partial sums of the
      // two frames after each pass (the out slot)
      const int slot = p.out_slot;
      ConvProblem cp = plain_problem(tail_x, nullptr, (int)Tall, tail_h, tail_w, c, 0, W_(st.sw), c, 1, 1, 1, F_(st.sb),
                                     nullptr, nullptr);
      cp.norm_gamma = F_(p.norm_out);
      cp.norm_eps = d->eps;
      cp.norm_silu = 1;
      cp.ntaps = 4;
      cp.phases = 4;
      cp.kh = 2;
      cp.kw = 2;
      cp.Ho = 2 * tail_h;
      cp.Wo = 2 * tail_w;
      cp.hmul = 2;
      cp.wmul = 2;
      cp.head_w = (const bf16_t*)W_(p.out_w);
      cp.head_b = F_(p.out_b);
      cp.head_co = d->out_channels;
      cp.video = (bf16_t*)video->data;
      cp.video_frames = video->t;
      cp.video_fbase = (int)fo;
      cp.carry = (float*)slot_ptr(slot);
      cp.carry_valid = cache->valid[slot] > 0 ? 1 : 0;
      const int64_t P_in = Tall * tail_h * tail_w;
      WVD_TRY(run_conv(cp, s, conv_flops(P_in * 4, c, 4LL * c) + conv_flops(P_in * 4, d->out_channels, 27LL * c)));
      cache->valid[slot] = (int)std::min<int64_t>(2, cache->valid[slot] + Tall);
      tail_x = nullptr;
      return WVD_OK;
    }
    const size_t in_frame = (size_t)tail_h * tail_w * c;
    for (int64_t f0 = 0; f0 < Tall; f0 += wl.tail_frames) {
      const int64_t m = std::min<int64_t>(wl.tail_frames, Tall - f0);
      WVD_TRY(run_phase_conv(tail_x + (size_t)f0 * in_frame, (int)m, tail_h, tail_w, c, W_(st.sw), F_(st.sb), ba, s,
                             F_(p.norm_out), d->eps));
      act = ba;
      zbuf = bx[cur ^ 1];
      T = m;
      WVD_TRY(run_head(fo + f0));
    }
    T = Tall;
    tail_x = nullptr;
    return WVD_OK;
  };
  if (split == L) {
    for (int si = 0; si < L; ++si) WVD_TRY(run_stage(si, bx[cur], nullptr));
    WVD_TRY(run_tail(frame_offset));
  } else {
    // the early stages for all n latent frames, the last of them upsampling into xm
    for (int si = 0; si < split; ++si) WVD_TRY(run_stage(si, bx[cur], si + 1 == split ? bxm : nullptr));
    const int H0 = H, W0 = Wd, c0 = c;
    int64_t t0 = 0, fo = frame_offset;
    for (int64_t l0 = 0; l0 < n; l0 += nh) {
      const int64_t m = std::min<int64_t>(nh, n - l0);
      const ChunkFrames fs = chunk_frames(d, m, rule && l0 == 0);
      T = fs.stage_in[split];
      H = H0;
      Wd = W0;
      c = c0;
      act = nullptr;
      zbuf = nullptr;
      stage_pre_act = false;  // (the split level's input comes from xm, never pre-activated)
      stage_sc_ready = false;
      const bf16_t* x = bxm + (size_t)t0 * H0 * W0 * c0;
      for (int si = split; si < L; ++si) {
        WVD_TRY(run_stage(si, x, nullptr));
        x = bx[cur];
      }
      WVD_TRY(run_tail(fo));
      t0 += T;
      fo += fs.video;
    }
  }
  cache->next_latent += n;
  cache->next_frame += fr.video;
  if (first) cache->rule = first_frame_rule != 0;
  return WVD_OK;
}

}  // namespace

extern "C" wvd_status wvd_decode_chunk(const wvd_decoder_desc* d, const void* packed, wvd_cache cache,
                                       const wvd_tensor* z, int first, int first_frame_rule, wvd_tensor* video,
                                       int64_t frame_offset, void* ws, size_t ws_bytes, wvd_stream stream) {
  return decode_chunk_impl(d, packed, cache, z, first, first_frame_rule, video, frame_offset, 0, ws, ws_bytes,
                           stream);
}

extern "C" wvd_status wvd_decode_chunk_split(const wvd_decoder_desc* d, const void* packed, wvd_cache cache,
                                             const wvd_tensor* z, int first, int first_frame_rule, wvd_tensor* video,
                                             int64_t frame_offset, int high_latent_frames, void* ws, size_t ws_bytes,
                                             wvd_stream stream) {
  return decode_chunk_impl(d, packed, cache, z, first, first_frame_rule, video, frame_offset, high_latent_frames, ws,
                           ws_bytes, stream);
}

// ==============================================================================================
// Timing
// ==============================================================================================
extern "C" wvd_status wvd_calib_dma_copy(const void* src, void* dst, size_t bytes, wvd_stream stream) {
  if (!src || !dst) return fail(WVD_ERR_ARG, "calib_dma_copy: null pointer");
  if (!aligned16(src) || !aligned16(dst) || bytes % 16) return fail(WVD_ERR_ALIGN, "calib_dma_copy: 16-byte multiples");
  const char* a = (const char*)src;
  const char* b = (const char*)dst;
  if (a < b + bytes && b < a + bytes) return fail(WVD_ERR_ARG, "calib_dma_copy: src and dst overlap");
  return hip_status(launch_dma_copy(src, dst, (int64_t)bytes, (hipStream_t)stream), "dma copy launch");
}

extern "C" wvd_status wvd_conv_force_config(int config) {
  if (config < -1 || config >= conv_config_count()) return fail(WVD_ERR_ARG, "conv config index out of range");
  g_force_config.store(config);
  return WVD_OK;
}

extern "C" wvd_status wvd_decode_fuse_norm1(int on) {
  g_fuse_norm1.store(on ? 1 : 0);
  return WVD_OK;
}

extern "C" wvd_status wvd_fuse_norm_shortcut(int on) {
  g_fuse_norm_sc.store(on ? 1 : 0);
  return WVD_OK;
}

extern "C" wvd_status wvd_decode_fuse_shortcut(int on) {
  g_fuse_shortcut.store(on ? 1 : 0);
  return WVD_OK;
}

extern "C" wvd_status wvd_decode_fuse_head(int on) {
  g_fuse_head.store(on ? 1 : 0);
  return WVD_OK;
}

extern "C" wvd_status wvd_conv_max_workgroups(int n) {
  if (n < 0) return fail(WVD_ERR_ARG, "negative workgroup cap");
  g_max_workgroups.store(n);
  return WVD_OK;
}

extern "C" wvd_status wvd_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.on = on != 0;
  return WVD_OK;
}

extern "C" wvd_status wvd_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (auto& r : g_timing.pending) {
    hipEventSynchronize(r.stop);
    g_timing.pool.push_back(r.start);
    g_timing.pool.push_back(r.stop);
  }
  g_timing.pending.clear();
  g_timing.launches.assign(conv_config_count(), 0);
  g_timing.ms.assign(conv_config_count(), 0.0);
  g_timing.flops.assign(conv_config_count(), 0.0);
  for (int k = 0; k < MEM_KINDS; ++k) {
    g_timing.mem_launches[k] = 0;
    g_timing.mem_ms[k] = 0.0;
    g_timing.mem_bytes[k] = 0.0;
  }
  g_timing.log.clear();
  return WVD_OK;
}

extern "C" int wvd_timing_read_mem(int i, const char** name, int64_t* launches, double* ms, double* bytes) {
  const char* nm = nullptr;
  wvd_timing_read(0, &nm, nullptr, nullptr, nullptr);  // drains the pending events
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (!name) return MEM_KINDS;
  if (i < 0 || i >= MEM_KINDS) return -1;
  *name = kMemKindNames[i];
  if (launches) *launches = g_timing.mem_launches[i];
  if (ms) *ms = g_timing.mem_ms[i];
  if (bytes) *bytes = g_timing.mem_bytes[i];
  return MEM_KINDS;
}

extern "C" int wvd_timing_launch(int i, int* config, double* ms, double* flops, int shape[10]) {
  const char* nm = nullptr;
  wvd_timing_read(0, &nm, nullptr, nullptr, nullptr);  // drains the pending events
  std::lock_guard<std::mutex> lk(g_timing.mu);
  const int n = (int)g_timing.log.size();
  if (i < 0 || i >= n) return n;
  const LaunchRecord& r = g_timing.log[i];
  if (config) *config = r.config;
  if (ms) *ms = r.ms;
  if (flops) *flops = r.flops;
  if (shape)
    for (int k = 0; k < 10; ++k) shape[k] = r.shape[k];
  return n;
}

extern "C" int wvd_timing_read(int i, const char** name, int64_t* launches, double* ms, double* flops) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  const int n = conv_config_count();
  if ((int)g_timing.launches.size() != n) {
    g_timing.launches.assign(n, 0);
    g_timing.ms.assign(n, 0.0);
    g_timing.flops.assign(n, 0.0);
  }
  for (auto& r : g_timing.pending) {
    float t = 0.0f;
    const bool got = hipEventSynchronize(r.stop) == hipSuccess && hipEventElapsedTime(&t, r.start, r.stop) == hipSuccess;
    if (got && r.mem >= 0 && r.mem < MEM_KINDS) {
      g_timing.mem_launches[r.mem] += 1;
      g_timing.mem_ms[r.mem] += t;
      g_timing.mem_bytes[r.mem] += r.flops;
    } else if (got && r.config >= 0 && r.config < n) {
      g_timing.launches[r.config] += 1;
      g_timing.ms[r.config] += t;
      g_timing.flops[r.config] += r.flops;
      LaunchRecord l{r.config, t, r.flops, {}};
      for (int k = 0; k < 10; ++k) l.shape[k] = r.shape[k];
      g_timing.log.push_back(l);
    }
    g_timing.pool.push_back(r.start);
    g_timing.pool.push_back(r.stop);
  }
  g_timing.pending.clear();
  if (!name) return n;
  if (i < 0 || i >= n) return -1;
  *name = conv_config_name(i);
  if (launches) *launches = g_timing.launches[i];
  if (ms) *ms = g_timing.ms[i];
  if (flops) *flops = g_timing.flops[i];
  return n;
}
