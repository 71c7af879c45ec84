// VALU throughput of gfx950 for the instruction mixes of the selective scan.
//
// The scan's prefill spends its time in the fp32 VALU: per channel-token and
// state it forms delta*A' (a multiply), the decay exp2 (v_exp_f32), the input
// term (delta*x)*B (a multiply), the state update (an FMA) and the output
// contribution C*h (an FMA).  These kernels measure how fast one MI355X issues
// each part on its own and in that mix, so that the ceiling the scan is held
// to rests on a measurement of this chip rather than on a vendor figure.
//
// Every kernel runs independent dependency chains per lane (enough of them to
// cover the pipeline latency) in a loop that the compiler cannot fold, over a
// grid that gives each SIMD several waves.  The host divides the number of
// VALU lane-instructions by the time between two events; the kernels also
// read the shader clock (s_memtime) and the fixed-frequency wall clock
// (s_memrealtime) so the rate can be stated per compute unit per clock.
//
// Plain fp32 only: the library is compiled with packed fp32 off, so no
// v_pk_* form appears (the ISA of these loops can be checked with
// --save-temps).

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "jscan_ubench.h"

namespace {

constexpr int kChains = 8;

struct Clocks {
  uint64_t t0, t1, w0, w1;
};

__device__ __forceinline__ void clocks_begin(Clocks* c) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    c->t0 = __builtin_amdgcn_s_memtime();
    c->w0 = __builtin_amdgcn_s_memrealtime();
  }
}
__device__ __forceinline__ void clocks_end(Clocks* c) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    c->t1 = __builtin_amdgcn_s_memtime();
    c->w1 = __builtin_amdgcn_s_memrealtime();
  }
}

// kChains FMA chains, `inner` FMAs each per outer iteration.
__global__ __launch_bounds__(256) void k_fma(float* out, Clocks* clk, int iters, float b, float c) {
  clocks_begin(clk);
  float v[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) v[k] = (float)(threadIdx.x + k) * 1e-3f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int k = 0; k < kChains; ++k) v[k] = fmaf(v[k], b, c);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += v[k];
  out[blockIdx.x * 256 + threadIdx.x] = s;
  __syncthreads();
  clocks_end(clk);
}

// kChains chains of v = exp2(-v): v stays in [0.5, 1].
__global__ __launch_bounds__(256) void k_exp(float* out, Clocks* clk, int iters) {
  clocks_begin(clk);
  float v[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) v[k] = (float)(threadIdx.x + k) * 1e-3f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int k = 0; k < kChains; ++k) v[k] = __builtin_amdgcn_exp2f(-v[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += v[k];
  out[blockIdx.x * 256 + threadIdx.x] = s;
  __syncthreads();
  clocks_end(clk);
}

// One exp chain step and four FMA chain steps per group, all independent:
// if the transcendental and the FMAs issued in parallel the group would cost
// the time of four FMAs, if not that of four FMAs plus one exp.
__global__ __launch_bounds__(256) void k_exp_fma(float* out, Clocks* clk, int iters, float b, float c) {
  clocks_begin(clk);
  float e[kChains / 2], f[2 * kChains];
#pragma unroll
  for (int k = 0; k < kChains / 2; ++k) e[k] = (float)(threadIdx.x + k) * 1e-3f;
#pragma unroll
  for (int k = 0; k < 2 * kChains; ++k) f[k] = (float)(threadIdx.x + k) * 1e-3f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int k = 0; k < kChains / 2; ++k) {
        e[k] = __builtin_amdgcn_exp2f(-e[k]);
#pragma unroll
        for (int j = 0; j < 4; ++j) f[4 * k + j] = fmaf(f[4 * k + j], b, c);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains / 2; ++k) s += e[k];
#pragma unroll
  for (int k = 0; k < 2 * kChains; ++k) s += f[k];
  out[blockIdx.x * 256 + threadIdx.x] = s;
  __syncthreads();
  clocks_end(clk);
}

// The scan's token step for 16 states: per state a multiply (dt * a2), an
// exp2, a multiply (dx * B), the state FMA and the output FMA, with B and C
// wave-uniform (kernel arguments, so SGPR operands as in the scan) and one
// FMA per token to vary dt and dx.
struct Rows { float a[16]; float B[16]; float C[16]; };

__global__ __launch_bounds__(256) void k_scan_mix(float* out, Clocks* clk, int iters, Rows r) {
  clocks_begin(clk);
  float h[16], a2[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    h[n] = 0.f;
    a2[n] = r.a[n] * (1.0f + (float)(threadIdx.x & 7) * 1e-3f);
  }
  float dt = 0.1f + (float)(threadIdx.x & 63) * 1e-4f, acc = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      dt = fmaf(dt, -0.5f, 0.15f);        // stays near 0.1: a fresh value per token
      const float dx = dt * 0.5f;
#pragma unroll
      for (int n = 0; n < 16; ++n) h[n] = fmaf(__builtin_amdgcn_exp2f(dt * a2[n]), h[n], dx * r.B[n]);
      float y = 0.f;
#pragma unroll
      for (int n = 0; n < 16; ++n) y = fmaf(r.C[n], h[n], y);
      acc += y;
    }
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc;
  __syncthreads();
  clocks_end(clk);
}

}  // namespace

extern "C" int jscan_ubench_valu(int kind, int64_t waves, int iters, double* seconds, double* lane_instr,
                                 double* trans_lane_instr, double* clock_mhz, double* wall_mhz) {
  if (waves <= 0 || waves % 4 != 0 || iters <= 0 || kind < 0 || kind > 3) return 1;
  const int64_t blocks = waves / 4;
  const int64_t lanes = blocks * 256;
  float* out = nullptr;
  Clocks* clk = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = 2;
  if (hipMalloc(&out, lanes * sizeof(float)) != hipSuccess) return 2;
  if (hipMalloc(&clk, sizeof(Clocks)) != hipSuccess) { (void)hipFree(out); return 2; }
  Rows rows;
  for (int n = 0; n < 16; ++n) {
    rows.a[n] = -1.4427f * (1.0f + n);
    rows.B[n] = 0.25f - 0.01f * n;
    rows.C[n] = 0.2f + 0.01f * n;
  }
  // lane-instructions per outer iteration (VALU, and transcendental among them)
  double per_iter = 0, per_iter_trans = 0;
  auto launch = [&]() {
    switch (kind) {
      case 0: hipLaunchKernelGGL(k_fma, dim3((unsigned)blocks), dim3(256), 0, 0, out, clk, iters, 0.999f, 1e-4f); break;
      case 1: hipLaunchKernelGGL(k_exp, dim3((unsigned)blocks), dim3(256), 0, 0, out, clk, iters); break;
      case 2: hipLaunchKernelGGL(k_exp_fma, dim3((unsigned)blocks), dim3(256), 0, 0, out, clk, iters, 0.999f, 1e-4f); break;
      default: hipLaunchKernelGGL(k_scan_mix, dim3((unsigned)blocks), dim3(256), 0, 0, out, clk, iters, rows); break;
    }
  };
  switch (kind) {
    case 0: per_iter = 16.0 * kChains; break;
    case 1: per_iter = per_iter_trans = 16.0 * kChains; break;
    case 2: per_iter = 4.0 * (kChains / 2) * 5; per_iter_trans = 4.0 * (kChains / 2); break;
    default: per_iter = 4.0 * (2 + 16 * 5 + 1); per_iter_trans = 4.0 * 16; break;
  }
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) goto done;
  launch();                                   // warm-up (clocks, code object)
  if (hipDeviceSynchronize() != hipSuccess) goto done;
  if (hipEventRecord(e0, 0) != hipSuccess) goto done;
  launch();
  if (hipEventRecord(e1, 0) != hipSuccess) goto done;
  if (hipEventSynchronize(e1) != hipSuccess) goto done;
  {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) goto done;
    Clocks c;
    if (hipMemcpy(&c, clk, sizeof(c), hipMemcpyDeviceToHost) != hipSuccess) goto done;
    int wall_khz = 0;
    if (hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, 0) != hipSuccess) goto done;
    *seconds = ms * 1e-3;
    *lane_instr = per_iter * (double)iters * (double)lanes;
    *trans_lane_instr = per_iter_trans * (double)iters * (double)lanes;
    *wall_mhz = wall_khz * 1e-3;
    const double wall_ticks = (double)(c.w1 - c.w0);
    *clock_mhz = wall_ticks > 0 ? (double)(c.t1 - c.t0) / wall_ticks * (*wall_mhz) : 0.0;
    rc = 0;
  }
done:
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(clk);
  (void)hipFree(out);
  return rc;
}
