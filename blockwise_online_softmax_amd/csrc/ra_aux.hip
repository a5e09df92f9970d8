// HBM-bound helper kernels of the ring-attention path: state init, finalize
// (out = acc / l, lse = m + ln l), layout permutation of rows and positions.
// Each is a grid-stride loop of coalesced 16-byte (or 4-byte) accesses whose
// grid covers the data in one pass where it can, with non-temporal accesses
// to the large streams (on MI355X a one-pass grid of 256-thread blocks
// streams at about 6.4 TB/s; a grid capped at 32 blocks per CU at 4.6-5.2).
#include "ra_internal.h"

namespace ra {

namespace {

constexpr int kThreads = 256;

inline unsigned grid_for(int64_t n) {
  int64_t g = (n + kThreads - 1) / kThreads;
  if (g < 1) g = 1;
  if (g > ((int64_t)1 << 30)) g = (int64_t)1 << 30;
  return (unsigned)g;
}

// Workgroups are dealt to the 8 XCDs (each with its own L2) round-robin.
// Renumber them so that each XCD takes one contiguous eighth of the data:
// per-row values that neighbouring workgroups share (m, l) then sit in one
// L2 instead of being fetched from HBM by several.
__device__ inline int64_t xcd_block() {
  const unsigned b = blockIdx.x, n = gridDim.x;
  if (n % 8 != 0) return b;
  return (int64_t)(b % 8) * (n / 8) + b / 8;
}

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

__device__ inline unsigned pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

// The empty running state ("Explain ring attention...", "The ring": max
// starts at -inf, sum and output at zero).
__global__ void state_init_kernel(float* __restrict__ m, float* __restrict__ l,
                                  float* __restrict__ acc, int64_t rows, int64_t D) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t i = t0; i < rows; i += stride) {
    m[i] = -__builtin_inff();
    l[i] = 0.f;
  }
  const int64_t n4 = rows * D / 4;
  f32x4* a4 = reinterpret_cast<f32x4*>(acc);
  for (int64_t i = t0; i < n4; i += stride)
    __builtin_nontemporal_store(f32x4{0.f, 0.f, 0.f, 0.f}, a4 + i);
}

// out = acc / l, lse = m + ln l; rows with l == 0 give out = 0, lse = -inf
// ("Module 23: Distributed Training", "The Math: One Block at a Time": divide
// at the end; "3.6 Distributed Training II", "Vocab-parallel cross-entropy":
// logsumexp = m + log Z).  One thread per 4 consecutive elements of a row.
template <int OUT_BF16>
__global__ void finalize_kernel(const float* __restrict__ m, const float* __restrict__ l,
                                const float* __restrict__ acc, void* __restrict__ out,
                                float* __restrict__ lse, int64_t rows, int qshift) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t n4 = rows << qshift;  // 2^qshift = D / 4 pieces per row
  const f32x4* a4 = reinterpret_cast<const f32x4*>(acc);
  for (int64_t i = xcd_block() * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const int64_t row = i >> qshift;
    const float lv = l[row];
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    if (lv > 0.f) {
      const float inv = 1.0f / lv;
      o = __builtin_nontemporal_load(a4 + i) * inv;
    }
    if (OUT_BF16) {
      u32x2 w = {pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w)};
      __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(out) + i);
    } else {
      __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(out) + i);
    }
    if (lse != nullptr && (i & ((1 << qshift) - 1)) == 0)
      lse[row] = lv > 0.f ? m[row] + logf(lv) : -__builtin_inff();
  }
}

// Row permutation between natural and device order; iterates over the
// device-ordered index so that one side is always read/written in order.
// I is the index type: 32-bit when the whole tensor has < 2^31 units (the
// divisions are then far cheaper), else 64-bit.
template <typename U, typename I>
__global__ void permute_kernel(const U* __restrict__ src, U* __restrict__ dst, int64_t outer,
                               int64_t S, int64_t upr, int N, int blk, int layout, int inverse) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const I per_outer = (I)(S * upr);
  const int64_t n = outer * (S * upr);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const I o = (I)i / per_outer;
    const I rem = (I)i - o * per_outer;
    const I di = rem / (I)upr;  // device-ordered row
    const I u = rem - di * (I)upr;
    const int p = (int)((uint32_t)di / (uint32_t)blk);
    const int a = (int)((uint32_t)di - (uint32_t)p * (uint32_t)blk);
    const int64_t ni = layout_pos(layout, N, blk, p, a);  // natural row
    const int64_t base = (int64_t)o * (S * upr);
    if (inverse)
      __builtin_nontemporal_store(__builtin_nontemporal_load(src + base + (int64_t)di * upr + u),
                                  dst + base + ni * upr + u);
    else
      __builtin_nontemporal_store(__builtin_nontemporal_load(src + base + ni * upr + u),
                                  dst + base + (int64_t)di * upr + u);
  }
}

__global__ void positions_kernel(int32_t* __restrict__ pos, int64_t count, int N, int blk,
                                 int layout, int device) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
    const int p = device < 0 ? (int)(i / blk) : device;
    const int a = device < 0 ? (int)(i - (int64_t)p * blk) : (int)i;
    pos[i] = layout_pos(layout, N, blk, p, a);
  }
}

}  // namespace

hipError_t launch_state_init(float* m, float* l, float* acc, int64_t rows, int64_t D,
                             hipStream_t s) {
  hipLaunchKernelGGL(state_init_kernel, dim3(grid_for(rows * D / 4)), dim3(kThreads), 0, s, m,
                     l, acc, rows, D);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* m, const float* l, const float* acc, void* out,
                           float* lse, int64_t rows, int64_t D, int out_dtype, hipStream_t s) {
  const dim3 g(grid_for(rows * D / 4));
  int qs = 0;  // D is a power of two from 8 to 128
  while (((int64_t)4 << qs) < D) ++qs;
  if (out_dtype == RA_BF16)
    hipLaunchKernelGGL(finalize_kernel<1>, g, dim3(kThreads), 0, s, m, l, acc, out, lse, rows, qs);
  else
    hipLaunchKernelGGL(finalize_kernel<0>, g, dim3(kThreads), 0, s, m, l, acc, out, lse, rows, qs);
  return hipGetLastError();
}

hipError_t launch_permute(const void* src, void* dst, int64_t outer, int64_t S, int64_t row_bytes,
                          int N, int layout, int inverse, hipStream_t s) {
  const int blk = (int)(S / N);
  const bool v16 = row_bytes % 16 == 0;
  const int64_t upr = row_bytes / (v16 ? 16 : 4);
  const int64_t n = outer * S * upr;
  const dim3 g(grid_for(n)), b(kThreads);
  const bool narrow = n < ((int64_t)1 << 31);
  if (v16 && narrow)
    hipLaunchKernelGGL((permute_kernel<u32x4, uint32_t>), g, b, 0, s, (const u32x4*)src,
                       (u32x4*)dst, outer, S, upr, N, blk, layout, inverse);
  else if (v16)
    hipLaunchKernelGGL((permute_kernel<u32x4, int64_t>), g, b, 0, s, (const u32x4*)src,
                       (u32x4*)dst, outer, S, upr, N, blk, layout, inverse);
  else if (narrow)
    hipLaunchKernelGGL((permute_kernel<unsigned, uint32_t>), g, b, 0, s, (const unsigned*)src,
                       (unsigned*)dst, outer, S, upr, N, blk, layout, inverse);
  else
    hipLaunchKernelGGL((permute_kernel<unsigned, int64_t>), g, b, 0, s, (const unsigned*)src,
                       (unsigned*)dst, outer, S, upr, N, blk, layout, inverse);
  return hipGetLastError();
}

hipError_t launch_positions(int32_t* pos, int64_t S, int N, int layout, int device,
                            hipStream_t s) {
  const int blk = (int)(S / N);
  const int64_t count = device < 0 ? S : blk;
  hipLaunchKernelGGL(positions_kernel, dim3(grid_for(count)), dim3(kThreads), 0, s, pos, count,
                     N, blk, layout, device);
  return hipGetLastError();
}

}  // namespace ra
