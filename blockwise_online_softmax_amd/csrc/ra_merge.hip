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
// One thread per 16 bytes of a row (4 fp32 or 8 bf16 elements); a row has
// at most 32 such pieces, so every row lies in one wavefront and all of its
// lanes read the row's m / l / lse before any lane writes them: `out` may be
// the same buffers as `a` or `b`.  The grid covers every piece in one pass
// where it can (measured on MI355X: a one-pass grid of 256-thread blocks with
// non-temporal 16-byte accesses streams fastest); the loop only serves sizes
// beyond 2^30 blocks.
#include "ra_internal.h"

namespace ra {

namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int kThreads = 256;

// Workgroups are dealt to the 8 XCDs (each with its own L2) round-robin.
// Renumber them so that each XCD takes one contiguous eighth of the rows:
// the per-row m / l / lse values that neighbouring workgroups share then sit
// in one L2 instead of being fetched from HBM by several.
__device__ inline int64_t xcd_block() {
  const unsigned b = blockIdx.x, n = gridDim.x;
  if (n % 8 != 0) return b;
  return (int64_t)(b % 8) * (n / 8) + b / 8;
}

__device__ inline unsigned pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}
// bf16 -> fp32 is exact: the 16 bits become the high half of the float
__device__ inline f32x4 unpack_lo(u32x4 w) {
  return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
               __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
}
__device__ inline f32x4 unpack_hi(u32x4 w) {
  return f32x4{__uint_as_float(w.z << 16), __uint_as_float(w.z & 0xffff0000u),
               __uint_as_float(w.w << 16), __uint_as_float(w.w & 0xffff0000u)};
}

// Weights of the two sides for one row: e^(xa - x) and e^(xb - x) with
// x = max(xa, xb); 0 for a side at -inf (also when both are).
__device__ inline void side_weights(float xa, float xb, float& x, float& wa, float& wb) {
  x = fmaxf(xa, xb);
  const bool none = x == -__builtin_inff();
  wa = none || xa == -__builtin_inff() ? 0.f : expf(xa - x);
  wb = none || xb == -__builtin_inff() ? 0.f : expf(xb - x);
}

// pieces: rows << pshift (2^pshift 16-byte pieces per row of acc)
__global__ void state_merge_kernel(const float* ma, const float* la, const float* acca,
                                   const float* mb, const float* lb, const float* accb,
                                   float* mo, float* lo, float* acco, int64_t pieces, int pshift) {
#pragma clang fp contract(off)
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = xcd_block() * blockDim.x + threadIdx.x; i < pieces; i += stride) {
    const int64_t row = i >> pshift;
    float m, wa, wb;
    side_weights(ma[row], mb[row], m, wa, wb);
    const float l = la[row] * wa + lb[row] * wb;
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(acca) + i);
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(accb) + i);
    __builtin_nontemporal_store(a * wa + b * wb, reinterpret_cast<f32x4*>(acco) + i);
    if ((i & ((1 << pshift) - 1)) == 0) {
      mo[row] = m;
      lo[row] = l;
    }
  }
}

template <bool BF16>
__global__ void out_merge_kernel(const void* oa, const float* lsea, const void* ob,
                                 const float* lseb, void* oo, float* lseo, int64_t pieces,
                                 int pshift) {
#pragma clang fp contract(off)
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = xcd_block() * blockDim.x + threadIdx.x; i < pieces; i += stride) {
    const int64_t row = i >> pshift;
    float x, wa, wb;
    side_weights(lsea[row], lseb[row], x, wa, wb);
    // weights are e^(lse_side - lse) = e^(lse_side - x) / (wa + wb)
    const float z = wa + wb;
    const float lse = z > 0.f ? x + logf(z) : -__builtin_inff();
    const float inv = z > 0.f ? 1.0f / z : 0.f;
    wa *= inv;
    wb *= inv;
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(oa) + i);
    const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ob) + i);
    u32x4 r;
    if (BF16) {
      const f32x4 lo4 = unpack_lo(a) * wa + unpack_lo(b) * wb;
      const f32x4 hi4 = unpack_hi(a) * wa + unpack_hi(b) * wb;
      r = u32x4{pack_bf16x2(lo4.x, lo4.y), pack_bf16x2(lo4.z, lo4.w), pack_bf16x2(hi4.x, hi4.y),
                pack_bf16x2(hi4.z, hi4.w)};
    } else {
      r = __builtin_bit_cast(u32x4, __builtin_bit_cast(f32x4, a) * wa +
                                        __builtin_bit_cast(f32x4, b) * wb);
    }
    __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(oo) + i);
    if ((i & ((1 << pshift) - 1)) == 0) lseo[row] = lse;
  }
}

// log2 of the 16-byte pieces in a row of D elements of `esize` bytes
// (D is a power of two from 8 to 128)
int piece_shift(int64_t D, int esize) {
  int s = 0;
  while (((int64_t)16 << s) < D * esize) ++s;
  return s;
}

unsigned grid_for(int64_t pieces) {
  const int64_t blocks = (pieces + kThreads - 1) / kThreads;
  const int64_t cap = (int64_t)1 << 30;
  return (unsigned)(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

}  // namespace

hipError_t launch_state_merge(const float* ma, const float* la, const float* acca,
                              const float* mb, const float* lb, const float* accb, float* mo,
                              float* lo, float* acco, int64_t rows, int64_t D, hipStream_t s) {
  const int ps = piece_shift(D, 4);
  const int64_t pieces = rows << ps;
  hipLaunchKernelGGL(state_merge_kernel, dim3(grid_for(pieces)), dim3(kThreads), 0, s, ma, la,
                     acca, mb, lb, accb, mo, lo, acco, pieces, ps);
  return hipGetLastError();
}

hipError_t launch_out_merge(const void* oa, const float* lsea, const void* ob, const float* lseb,
                            void* oo, float* lseo, int64_t rows, int64_t D, int dtype,
                            hipStream_t s) {
  const bool bf16 = dtype == RA_BF16;
  const int ps = piece_shift(D, bf16 ? 2 : 4);
  const int64_t pieces = rows << ps;
  const dim3 g(grid_for(pieces)), b(kThreads);
  if (bf16)
    hipLaunchKernelGGL(out_merge_kernel<true>, g, b, 0, s, oa, lsea, ob, lseb, oo, lseo, pieces,
                       ps);
  else
    hipLaunchKernelGGL(out_merge_kernel<false>, g, b, 0, s, oa, lsea, ob, lseb, oo, lseo, pieces,
                       ps);
  return hipGetLastError();
}

}  // namespace ra
