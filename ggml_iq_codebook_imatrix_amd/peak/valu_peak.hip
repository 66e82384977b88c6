// valu_peak.hip -- measured VALU ceiling for the encoder's roofline.
//
// The encoder's search is priced in algorithmic ops (an FMA, a MUL and a MIN
// count one op each; a 3-input min retires two).  This library measures what
// one MI355X sustains for the three instruction forms the search is made of,
// under the same build as the encoder (contraction off, packed fp32 disabled):
//   mode 0  fp32 FMA with every operand in a VGPR (the candidate FMAs)
//   mode 1  3-input fp32 min (the running minima)
//   mode 2  the candidate stage's mix: two FMAs, then one 3-input min folding
//           both into a running minimum (4 ops per 3 instructions)
// Independent chains (8 per lane), 8 waves per SIMD on every CU.  The first
// workgroup records the shader clock counter and the constant-rate wall
// counter around its work, which gives the clock the chip ran at.
// Measurement support only: not part of libiq's C ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kChains = 8;

template <int MODE>
__global__ void __launch_bounds__(256) valu_kernel(float *out, int iters, float seed, unsigned long long *clocks) {
  float acc[kChains], a[kChains], b[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) {
    acc[k] = MODE == 0 ? 0.0f : 1e30f;
    a[k] = seed + static_cast<float>(threadIdx.x) * 1e-3f + static_cast<float>(k);
    b[k] = seed * 0.5f + static_cast<float>(k) * 1e-2f;
  }
  unsigned long long c0 = 0, w0 = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    c0 = clock64();
    w0 = wall_clock64();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) {
      if (MODE == 0) {
        acc[k] = __builtin_fmaf(a[k], b[(k + 1) % kChains], acc[k]);
      } else if (MODE == 1) {  // a neighbouring chain as the second input: nothing loop invariant
        acc[k] = fminf(fminf(acc[k], acc[(k + 1) % kChains]), b[(k + 3) % kChains]);
      } else {  // both candidates depend on the chain, so nothing is loop invariant
        const float t0 = __builtin_fmaf(acc[k], b[(k + 1) % kChains], a[k]);
        const float t1 = __builtin_fmaf(acc[k], b[(k + 2) % kChains], a[(k + 3) % kChains]);
        acc[k] = fminf(fminf(acc[k], t0), t1);
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += acc[k];
  out[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clocks[0] = clock64() - c0;
    clocks[1] = wall_clock64() - w0;
  }
}

}  // namespace

// ops_per_s: algorithmic ops per second over the whole device (FMA 1, min3 2);
// instr_per_s: VALU instructions per second counted as one per lane;
// clock_hz: shader clock during the run (0 if the counters are unavailable).
// Returns 0, or -1 on a HIP error or an unknown mode.
extern "C" int valu_peak(int mode, int iters, double *ops_per_s, double *instr_per_s, double *clock_hz) {
  if (mode < 0 || mode > 2 || iters < 1 || !ops_per_s || !instr_per_s || !clock_hz) return -1;
  int dev = 0, cus = 0, wall_khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev);
  if (cus < 1) return -1;
  const int threads = 256, blocks = cus * 8;  // 8 waves per SIMD: 32 waves per CU
  float *out = nullptr;
  unsigned long long *clk = nullptr;
  if (hipMalloc(&out, sizeof(float) * blocks * threads) != hipSuccess) return -1;
  if (hipMalloc(&clk, 2 * sizeof(unsigned long long)) != hipSuccess) { hipFree(out); return -1; }
  hipEvent_t e0, e1;
  hipEventCreate(&e0);
  hipEventCreate(&e1);
  auto launch = [&](int n) {
    if (mode == 0) hipLaunchKernelGGL(valu_kernel<0>, dim3(blocks), dim3(threads), 0, 0, out, n, 1.0f, clk);
    else if (mode == 1) hipLaunchKernelGGL(valu_kernel<1>, dim3(blocks), dim3(threads), 0, 0, out, n, 1.0f, clk);
    else hipLaunchKernelGGL(valu_kernel<2>, dim3(blocks), dim3(threads), 0, 0, out, n, 1.0f, clk);
  };
  launch(iters / 4 + 1);  // warm the clocks
  hipEventRecord(e0, 0);
  launch(iters);
  hipEventRecord(e1, 0);
  const bool ok = hipEventSynchronize(e1) == hipSuccess && hipGetLastError() == hipSuccess;
  float ms = 0.0f;
  hipEventElapsedTime(&ms, e0, e1);
  unsigned long long c[2] = {0, 0};
  hipMemcpy(c, clk, sizeof(c), hipMemcpyDeviceToHost);
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  hipFree(out);
  hipFree(clk);
  if (!ok || ms <= 0.0f) return -1;
  const double lanes = static_cast<double>(blocks) * threads * iters * kChains;
  const double instr = mode == 2 ? 3.0 : 1.0, ops = mode == 0 ? 1.0 : mode == 1 ? 2.0 : 4.0;
  *ops_per_s = lanes * ops / (ms * 1e-3);
  *instr_per_s = lanes * instr / (ms * 1e-3);
  *clock_hz = (wall_khz > 0 && c[1] > 0) ? static_cast<double>(c[0]) / (static_cast<double>(c[1]) / (wall_khz * 1e3))
                                          : 0.0;
  return 0;
}

namespace {
// One wave reads the shader clock counter and the constant-rate wall counter
// across a fixed stretch of wall time.
__global__ void clock_kernel(unsigned long long wall_ticks, unsigned long long *clocks) {
  const unsigned long long c0 = clock64(), w0 = wall_clock64();
  unsigned long long w = w0;
  while (w - w0 < wall_ticks) w = wall_clock64();
  if (threadIdx.x == 0) {
    clocks[0] = clock64() - c0;
    clocks[1] = w - w0;
  }
}
}  // namespace

// clock_hz: the shader clock over `us` microseconds of a one-wave kernel
// launched on the null stream now (so it reads the clock the chip runs at
// right after the work queued before it).  Returns 0, or -1 on a HIP error.
extern "C" int shader_clock(int us, double *clock_hz) {
  if (us < 1 || !clock_hz) return -1;
  int dev = 0, wall_khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev);
  if (wall_khz <= 0) return -1;
  unsigned long long *clk = nullptr;
  if (hipMalloc(&clk, 2 * sizeof(unsigned long long)) != hipSuccess) return -1;
  const unsigned long long ticks = static_cast<unsigned long long>(wall_khz) * us / 1000;
  hipLaunchKernelGGL(clock_kernel, dim3(1), dim3(64), 0, 0, ticks, clk);
  unsigned long long c[2] = {0, 0};
  const bool ok = hipGetLastError() == hipSuccess && hipMemcpy(c, clk, sizeof(c), hipMemcpyDeviceToHost) == hipSuccess;
  hipFree(clk);
  if (!ok || c[1] == 0) return -1;
  *clock_hz = static_cast<double>(c[0]) / (static_cast<double>(c[1]) / (wall_khz * 1e3));
  return 0;
}
