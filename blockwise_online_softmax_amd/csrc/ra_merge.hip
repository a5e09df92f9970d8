// Merge of two partial attention results over disjoint key sets (HBM-bound).
//
// The fold of key blocks into a row's state does not depend on their order
// ("Module 23: Distributed Training", "The Math: One Block at a Time"), so two
// states built from disjoint key sets combine like one more fold: with
// m = max(ma, mb),
//   l = la e^(ma-m) + lb e^(mb-m),   acc = acca e^(ma-m) + accb e^(mb-m).
// On finalized results the same step is a log-sum-exp merge ("3.6
// Distributed Training II", "Vocab-parallel cross-entropy": logsumexp = m +
// log Z): lse = log(e^lse_a + e^lse_b), out = out_a e^(lse_a-lse) +
// out_b e^(lse_b-lse).  A side that saw no key (m = -inf, l = 0, or lse = -inf)
// contributes nothing; a row empty on both sides stays empty.
//
// Products are rounded before the sum (no fused multiply-add), so merging a
// with b and b with a give the same bits.
//
// One thread per 4 elements of a row; D/4 divides 64, so every row lies in one
// wavefront and all of its lanes read the row's m / l / lse before any lane
// writes them: `out` may be the same buffers as `a` or `b`.
#include "ra_internal.h"

namespace ra {

namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int kThreads = 256;

__device__ inline unsigned pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}
__device__ inline f32x4 unpack_bf16x4(u32x2 w) {
  // bf16 -> fp32 is exact: the 16 bits become the high half of the float
  return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
               __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
}

// Weights of the two sides for one row: e^(xa - x) and e^(xb - x) with
// x = max(xa, xb); 0 for a side at -inf (also when both are).
__device__ inline void side_weights(float xa, float xb, float& x, float& wa, float& wb) {
  x = fmaxf(xa, xb);
  const bool none = x == -__builtin_inff();
  wa = none || xa == -__builtin_inff() ? 0.f : expf(xa - x);
  wb = none || xb == -__builtin_inff() ? 0.f : expf(xb - x);
}

__global__ void state_merge_kernel(const float* ma, const float* la, const float* acca,
                                   const float* mb, const float* lb, const float* accb,
                                   float* mo, float* lo, float* acco, int64_t rows, int qshift) {
#pragma clang fp contract(off)
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t n4 = rows << qshift;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const int64_t row = i >> qshift;
    float m, wa, wb;
    side_weights(ma[row], mb[row], m, wa, wb);
    const float l = la[row] * wa + lb[row] * wb;
    const f32x4 a = reinterpret_cast<const f32x4*>(acca)[i];
    const f32x4 b = reinterpret_cast<const f32x4*>(accb)[i];
    reinterpret_cast<f32x4*>(acco)[i] = a * wa + b * wb;
    if ((i & ((1 << qshift) - 1)) == 0) {
      mo[row] = m;
      lo[row] = l;
    }
  }
}

template <bool BF16>
__global__ void out_merge_kernel(const void* oa, const float* lsea, const void* ob,
                                 const float* lseb, void* oo, float* lseo, int64_t rows,
                                 int qshift) {
#pragma clang fp contract(off)
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t n4 = rows << qshift;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const int64_t row = i >> qshift;
    float x, wa, wb;
    side_weights(lsea[row], lseb[row], x, wa, wb);
    // weights are e^(lse_side - lse) = e^(lse_side - x) / (wa + wb)
    const float z = wa + wb;
    const float lse = z > 0.f ? x + logf(z) : -__builtin_inff();
    const float inv = z > 0.f ? 1.0f / z : 0.f;
    wa *= inv;
    wb *= inv;
    f32x4 a, b;
    if (BF16) {
      a = unpack_bf16x4(reinterpret_cast<const u32x2*>(oa)[i]);
      b = unpack_bf16x4(reinterpret_cast<const u32x2*>(ob)[i]);
    } else {
      a = reinterpret_cast<const f32x4*>(oa)[i];
      b = reinterpret_cast<const f32x4*>(ob)[i];
    }
    const f32x4 o = a * wa + b * wb;
    if (BF16)
      reinterpret_cast<u32x2*>(oo)[i] = u32x2{pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w)};
    else
      reinterpret_cast<f32x4*>(oo)[i] = o;
    if ((i & ((1 << qshift) - 1)) == 0) lseo[row] = lse;
  }
}

// log2(D / 4); D is a power of two from 8 to 128
int quad_shift(int64_t D) {
  int s = 0;
  while ((int64_t)4 << s < D) ++s;
  return s;
}

unsigned grid_for(int64_t n4) {
  const int64_t blocks = (n4 + kThreads - 1) / kThreads;
  return (unsigned)(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

}  // namespace

hipError_t launch_state_merge(const float* ma, const float* la, const float* acca,
                              const float* mb, const float* lb, const float* accb, float* mo,
                              float* lo, float* acco, int64_t rows, int64_t D, hipStream_t s) {
  hipLaunchKernelGGL(state_merge_kernel, dim3(grid_for(rows * (D / 4))), dim3(kThreads), 0, s,
                     ma, la, acca, mb, lb, accb, mo, lo, acco, rows, quad_shift(D));
  return hipGetLastError();
}

hipError_t launch_out_merge(const void* oa, const float* lsea, const void* ob, const float* lseb,
                            void* oo, float* lseo, int64_t rows, int64_t D, int dtype,
                            hipStream_t s) {
  const dim3 g(grid_for(rows * (D / 4))), b(kThreads);
  const int qs = quad_shift(D);
  if (dtype == RA_BF16)
    hipLaunchKernelGGL(out_merge_kernel<true>, g, b, 0, s, oa, lsea, ob, lseb, oo, lseo, rows, qs);
  else
    hipLaunchKernelGGL(out_merge_kernel<false>, g, b, 0, s, oa, lsea, ob, lseb, oo, lseo, rows, qs);
  return hipGetLastError();
}

}  // namespace ra
