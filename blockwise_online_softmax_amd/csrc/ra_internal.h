// Internal declarations shared by the HIP kernels and the C-ABI layer of
// libra.so.  Not part of the public ABI (include/ra.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra.h"

namespace ra {

// Global position of local index `a` on device `dev` for a layout of S = N*blk
// tokens (zigzag chunk c = blk/2).  Layout statements: "Module 23: Distributed
// Training", "The Causal Imbalance -- and the Striped Fix" (striped: device p
// holds p, p+N, ...; zigzag named there); "Explain ring attention...", "The
// ring" (contiguous).  Zigzag reading: chunk p then chunk 2N-1-p.
__host__ __device__ inline int layout_pos(int layout, int N, int blk, int dev, int a) {
  if (layout == RA_STRIPED) return dev + a * N;
  if (layout == RA_ZIGZAG) {
    const int c = blk >> 1;
    return a < c ? dev * c + a : (2 * N - 1 - dev) * c + (a - c);
  }
  return dev * blk + a;
}

// How key/query positions reach an attention kernel.
enum PosMode : int {
  POS_NONE = 0,      // no mask: positions unused
  POS_ANALYTIC = 1,  // device-ordered data; position = layout_pos(layout, ...)
  POS_ARRAY = 2,     // explicit int32 arrays q_pos / k_pos, any order
};

// One launch of an attention kernel.  The query side is `nqblk` blocks of
// `qlen` rows (block i belongs to device dev0 + i); the key side is `nkblk`
// blocks of `klen` keys.  The query block of device p visits key blocks in
// ring order j = (p - s) mod nkblk, s = 0..nkblk-1.
struct AttnParams {
  const void* Q;   // [B, Hq, Sq_tot, D]
  const void* K;   // [B, Hkv, Sk_tot, D]
  const void* V;   // [B, Hkv, Sk_tot, D]
  const int32_t* q_pos;  // POS_ARRAY: [Sq_tot]
  const int32_t* k_pos;  // POS_ARRAY: [Sk_tot]
  float* m;        // state, [B, Hq, Sq_tot]       (state-in/out kernels)
  float* l;        // state, [B, Hq, Sq_tot]
  float* acc;      // state, [B, Hq, Sq_tot, D]
  void* out;       // [B, Hq, Sq_tot, D] Q's dtype  (fused-finalize kernels)
  float* lse;      // [B, Hq, Sq_tot]
  int64_t Sq_tot, Sk_tot;
  int B, Hq, Hkv;
  int nqblk, qlen, dev0;
  int nkblk, klen;
  int ntq;         // query tiles per query block (kernel specific)
  int layout, N, blk;  // POS_ANALYTIC
  float scale;     // score scale
  float sl2;       // scale * log2(e)
};

// Launchers (return hipGetLastError() after the launch).
// natural: a whole ring whose Q, K, V, out, lse are in natural token order
// (striped / zigzag rows addressed through the layout map, no permutes).
hipError_t launch_attn_mfma(const AttnParams& p, int D, bool causal, int pos_mode, bool state_io,
                            bool natural, hipStream_t s);
bool mfma_supports(int D);
hipError_t launch_attn_valu(const AttnParams& p, int D, int dtype, bool causal, int pos_mode,
                            bool state_io, hipStream_t s);
hipError_t launch_state_init(float* m, float* l, float* acc, int64_t rows, int64_t D,
                             hipStream_t s);
hipError_t launch_finalize(const float* m, const float* l, const float* acc, void* out,
                           float* lse, int64_t rows, int64_t D, int out_dtype, hipStream_t s);
hipError_t launch_permute(const void* src, void* dst, int64_t outer, int64_t S, int64_t row_bytes,
                          int N, int layout, int inverse, hipStream_t s);
hipError_t launch_positions(int32_t* pos, int64_t S, int N, int layout, int device,
                            hipStream_t s);
hipError_t launch_state_merge(const float* ma, const float* la, const float* acca,
                              const float* mb, const float* lb, const float* accb, float* mo,
                              float* lo, float* acco, int64_t rows, int64_t D, hipStream_t s);
hipError_t launch_ce_stats(const void* logits, int64_t ld, const int64_t* target, int64_t N,
                           int64_t V_loc, int64_t start0, int t, int dtype, float* m, float* s,
                           float* p, hipStream_t st);
int64_t ce_partial_count(int64_t N);
hipError_t launch_ce_combine(const float* m, const float* s, const float* p, int t, int64_t N,
                             float* loss, float* lse, float* partial, float* mean, hipStream_t st);
hipError_t launch_ce_grad(const void* logits, int64_t ld, const int64_t* target, const float* lse,
                          int64_t N, int64_t V_loc, int64_t start0, int t, float scale, int dtype,
                          void* grad, int64_t ldg, hipStream_t st);
hipError_t launch_out_merge(const void* oa, const float* lsea, const void* ob, const float* lseb,
                            void* oo, float* lseo, int64_t rows, int64_t D, int dtype,
                            hipStream_t s);

}  // namespace ra
