// Measurement kernel for bench.py, built into its own library (libra_probe.so),
// apart from the attention library: the sustained bf16 matrix-core rate of
// this GPU and the shader clock it runs at under that load.  The attention
// kernel's roofline fraction is quoted against the published peak; this
// gives the ceiling the hardware reaches in practice beside it.
//
// Every wavefront issues `iters` rounds of four independent
// v_mfma_f32_32x32x16_bf16 (32 x 32 x 16 x 2 = 32768 FLOP each) on register
// operands (random-looking bf16 or small constants); 512-thread workgroups (two wavefronts per SIMD, as the 8-wave
// attention kernel runs).  The first wavefront of each workgroup records
// the shader-clock counter (s_memtime) and the constant-rate counter
// (s_memrealtime) around its loop, so clock = d(memtime) / d(realtime) x
// the constant counter's rate.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

// A roughly normal value (sum of four uniforms, centred) from a hash of the
// element index: the MFMA's power, and with it the clock, depends on how many
// operand bits toggle, so the operands look like N(0,1) data, not constants.
__device__ inline float hash_normal(unsigned x) {
  float acc = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    acc += (float)(x & 0xffffu) * (1.0f / 65536.0f);
  }
  return (acc - 2.0f) * 1.7320508f;
}

template <bool RANDOM>
__global__ __launch_bounds__(512) void mfma_ceiling_kernel(int iters, float* sink,
                                                           unsigned long long* clk) {
  bf16x8 a, b;
  const unsigned gid = blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = RANDOM ? (__bf16)hash_normal(gid * 16 + i) : (__bf16)(float)((threadIdx.x + i) & 3);
    b[i] = RANDOM ? (__bf16)hash_normal(gid * 16 + 8 + i) : (__bf16)(float)((threadIdx.x * 3 + i) & 1);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  unsigned long long t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = __builtin_readcyclecounter();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  if (threadIdx.x == 0) {
    const unsigned long long t1 = __builtin_readcyclecounter();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (s == 12345.678f) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the MFMAs live
}

}  // namespace

extern "C" {

// Runs `wgs` workgroups x `iters` rounds on `stream`, returns 0 or a HIP error
// code.  random != 0: operands drawn like N(0,1) data; 0: small constants.
// sink: >= wgs * 512 floats, clk: 2 * wgs uint64 (device buffers,
// caller-owned); *ms: the launch's elapsed time (HIP events); *wall_khz: the
// rate of the s_memrealtime counter.
int ra_probe_mfma(int wgs, int iters, int random, float* sink, unsigned long long* clk, float* ms,
                  int* wall_khz, void* stream) {
  if (wgs < 1 || iters < 1 || sink == nullptr || clk == nullptr || ms == nullptr ||
      wall_khz == nullptr)
    return (int)hipErrorInvalidValue;
  hipStream_t s = (hipStream_t)stream;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(wall_khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return (int)e;
  hipEvent_t ev0, ev1;
  if ((e = hipEventCreate(&ev0)) != hipSuccess) return (int)e;
  if ((e = hipEventCreate(&ev1)) != hipSuccess) {
    hipEventDestroy(ev0);
    return (int)e;
  }
  hipEventRecord(ev0, s);
  if (random)
    hipLaunchKernelGGL(mfma_ceiling_kernel<true>, dim3(wgs), dim3(512), 0, s, iters, sink, clk);
  else
    hipLaunchKernelGGL(mfma_ceiling_kernel<false>, dim3(wgs), dim3(512), 0, s, iters, sink, clk);
  e = hipGetLastError();
  hipEventRecord(ev1, s);
  if (e == hipSuccess) e = hipEventSynchronize(ev1);
  if (e == hipSuccess) e = hipEventElapsedTime(ms, ev0, ev1);
  hipEventDestroy(ev0);
  hipEventDestroy(ev1);
  return (int)e;
}

}  // extern "C"
