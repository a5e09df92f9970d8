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

// Timing probe of the attention tile loop's instruction mix, without its
// copies, barriers, masks or causal walk: every wavefront issues `iters`
// rounds of NL LDS operand reads (alternately one 16-byte read of a K-like row
// and two transpose reads of a V-like tile, with the attention kernel's
// swizzles, so that no read has a bank conflict), each read feeding R MFMAs
// (R = 2: the read is shared by two 32-row query blocks, as 64 query rows per
// wave would share it), plus SM softmax units per MFMA (an FMA, an
// exponential and an add on independent registers).  LDSON = false feeds the
// MFMAs from registers instead.  The LDS holds data-like bf16 values, so the
// matrix cores toggle as many bits as on real data.
template <int W, int NL, int R, int SM, bool LDSON>
__global__ __launch_bounds__(W * 64, 1) void tile_mix_kernel(int iters, float* sink) {
  typedef __attribute__((address_space(3))) char lds_t;
  typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
  typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
  typedef __attribute__((ext_vector_type(4))) short i16x4;
  __shared__ __attribute__((aligned(1024))) char lds[65536];
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 65536 / 2; i += W * 64)
    ((__bf16*)lds)[i] = (__bf16)hash_normal((unsigned)i * 2654435761u + 7u);
  __syncthreads();
  u32x4 bq[2];
  for (int r = 0; r < 2; ++r)
    for (int c = 0; c < 4; ++c) {
      bf16x8 t;
      for (int i = 0; i < 8; ++i) t[i] = (__bf16)hash_normal((blockIdx.x * 512 + threadIdx.x) * 64 + r * 8 + i + c);
      bq[r][c] = __builtin_bit_cast(u32x4, t)[c];
    }
  const u32x4 areg = {bq[0].y ^ 1u, bq[1].x, bq[0].w, bq[1].z};
  f32x16 acc[4] = {};
  float x[32];
  for (int i = 0; i < 32; ++i) x[i] = 0.01f * (i + 1) + lane * 1e-3f;
  float sacc[4] = {0.f, 0.f, 0.f, 0.f};
  const lds_t* L = (const lds_t*)lds;
  const int r32 = lane & 31, hi = lane >> 5;
  const int kofs = r32 * 256 + ((hi ^ (r32 & 15)) << 4);  // K: row r, unit 2c + hi
  const int vkey = 4 * hi + ((lane & 15) >> 2);
  const int vu = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int vofs = vkey * 256 + ((vu ^ (4 * (vkey & 3))) << 4) + ((lane & 1) << 3);
  for (int it = 0; it < iters; ++it) {
    const int sw = (it & 1) << 13;  // alternate 8 KB halves (all reads in bounds)
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      u32x4 a;
      if constexpr (LDSON) {
        if (l & 1) {
          const lds_t* p = L + 32768 + sw + (vofs ^ (((l >> 1) & 3) << 6));
          const u32x2 a0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                         (__attribute__((address_space(3))) i16x4*)p));
          const u32x2 a1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                         (__attribute__((address_space(3))) i16x4*)(p + 8 * 256)));
          a = u32x4{a0.x, a0.y, a1.x, a1.y};
        } else {
          a = *(const __attribute__((address_space(3))) u32x4*)(L + sw + (kofs ^ (((l >> 1) & 7) << 5)));
        }
      } else {
        a = areg;
        a.x ^= (unsigned)l;
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int m = l * R + r;
        acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                             __builtin_bit_cast(bf16x8, bq[r]),
                                                             acc[m & 3], 0, 0, 0);
#pragma unroll
        for (int u = 0; u < SM; ++u) {
          const int e = (m * SM + u) & 31;
          x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], -0.7f, 0.3f));
          sacc[e & 3] += x[e];
        }
      }
    }
  }
  float s = 0.f;
  for (int j = 0; j < 4; ++j)
    for (int i = 0; i < 16; ++i) s += acc[j][i];
  for (int i = 0; i < 32; ++i) s += x[i];
  for (int i = 0; i < 4; ++i) s += sacc[i];
  if (s == 12345.678f) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the work live
}

template <int W, int NL, int R, int SM, bool LDSON>
hipError_t launch_mix(int wgs, int iters, float* sink, hipStream_t s) {
  hipLaunchKernelGGL((tile_mix_kernel<W, NL, R, SM, LDSON>), dim3(wgs), dim3(W * 64), 0, s, iters,
                     sink);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// The tile-mix probe (tile_mix_kernel) in configuration `cfg`: 0 MFMA only
// (8 waves), 1 MFMA + softmax (8 waves), 2 MFMA + 1 KB LDS operand per MFMA
// (8 waves), 3 the same + softmax (the 8-wave ring kernel's mix), 4 MFMA +
// 0.5 KB LDS per MFMA + softmax (4 waves of 64 query rows).  One workgroup
// per CU (`wgs` of them), `iters` rounds of 8 operand reads; returns 0 or a
// HIP error; *ms: elapsed time (HIP events); *mfma_per_wg: MFMAs one
// workgroup issues.  sink: >= wgs * 512 floats (device, caller-owned).
int ra_probe_tile_mix(int cfg, int wgs, int iters, float* sink, float* ms, long long* mfma_per_wg,
                      void* stream) {
  if (cfg < 0 || cfg > 4 || wgs < 1 || iters < 1 || sink == nullptr || ms == nullptr ||
      mfma_per_wg == nullptr)
    return (int)hipErrorInvalidValue;
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t ev0, ev1;
  hipError_t e;
  if ((e = hipEventCreate(&ev0)) != hipSuccess) return (int)e;
  if ((e = hipEventCreate(&ev1)) != hipSuccess) {
    hipEventDestroy(ev0);
    return (int)e;
  }
  hipEventRecord(ev0, s);
  switch (cfg) {
    case 0: e = launch_mix<8, 8, 1, 0, false>(wgs, iters, sink, s); break;
    case 1: e = launch_mix<8, 8, 1, 1, false>(wgs, iters, sink, s); break;
    case 2: e = launch_mix<8, 8, 1, 0, true>(wgs, iters, sink, s); break;
    case 3: e = launch_mix<8, 8, 1, 1, true>(wgs, iters, sink, s); break;
    default: e = launch_mix<4, 8, 2, 1, true>(wgs, iters, sink, s); break;
  }
  *mfma_per_wg = (long long)iters * 8 * (cfg == 4 ? 2 * 4 : 8);
  hipEventRecord(ev1, s);
  if (e == hipSuccess) e = hipEventSynchronize(ev1);
  if (e == hipSuccess) e = hipEventElapsedTime(ms, ev0, ev1);
  hipEventDestroy(ev0);
  hipEventDestroy(ev1);
  return (int)e;
}

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
