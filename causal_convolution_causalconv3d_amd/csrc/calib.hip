// Measurement support: a device copy that reads through the conv kernels' own load path.
//
// The conv kernels stage their operands with buffer loads that write LDS directly, 16 bytes per
// lane. Hardware byte counters (FETCH_SIZE, WRITE_SIZE) are converted to bytes with a factor
// measured on a copy of known size; this copy moves its data with exactly those instructions
// (each wave fetches 1 KB into its own LDS area, waits for it, reads it back with 16-byte LDS
// reads and stores it with 16-byte global stores), so the factor for that load path can be
// compared with the one measured on a plain elementwise copy.
#include "common.h"

namespace wvd {

namespace {

constexpr int kCalibWaves = 4;
constexpr int kCalibLoads = 4;  // 1 KB fetches in flight per wave

__global__ __launch_bounds__(kCalibWaves * 64) void dma_copy_kernel(const uint4* __restrict__ src,
                                                                    uint4* __restrict__ dst, int64_t n16) {
  typedef __attribute__((address_space(3))) void lds_void;
  __shared__ __attribute__((aligned(16))) uint4 stage[kCalibWaves][kCalibLoads][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // one wave step covers kCalibLoads * 64 chunks of 16 bytes
  const int64_t per_step = (int64_t)kCalibLoads * 64;
  const int64_t nwave = (int64_t)gridDim.x * kCalibWaves;
  for (int64_t base = ((int64_t)blockIdx.x * kCalibWaves + wave) * per_step; base < n16; base += nwave * per_step) {
    // the resource covers [base, n16): chunks past the end read as zero and are not stored
    const int64_t left = n16 - base;
    const int range = (int)((left < per_step ? left : per_step) * 16);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)(src + base), (short)0, range, 0x00020000);
#pragma unroll
    for (int k = 0; k < kCalibLoads; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)&stage[wave][k][0], 16, (k * 64 + lane) * 16, 0, 0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's fetches are in LDS
    asm volatile("" ::: "memory");
#pragma unroll
    for (int k = 0; k < kCalibLoads; ++k) {
      const int64_t i = base + k * 64 + lane;
      const uint4 v = stage[wave][k][lane];
      if (i < n16) dst[i] = v;
    }
    asm volatile("" ::: "memory");
  }
}

}  // namespace

hipError_t launch_dma_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0) return hipSuccess;
  const int64_t steps = (n16 + kCalibLoads * 64 - 1) / (kCalibLoads * 64);
  int64_t blocks = (steps + kCalibWaves - 1) / kCalibWaves;
  if (blocks > 256 * 8) blocks = 256 * 8;
  hipLaunchKernelGGL(dma_copy_kernel, dim3((unsigned)blocks), dim3(kCalibWaves * 64), 0, s, (const uint4*)src,
                     (uint4*)dst, n16);
  return hipGetLastError();
}

}  // namespace wvd
