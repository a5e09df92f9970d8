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

// Work split of one launch over the GPU's 8 XCDs (the compute dies, each with
// its own L2).  The hardware hands workgroup w to XCD w % 8 as that XCD's slot
// w / 8.  Work items are numbered XCD-major: XCD x owns items x*M .. x*M+M-1,
// longest first.  XCD x first runs entries dbeg[x] .. dbeg[x]+dcnt[x]-1 of the
// donated list (the first M - keep[y] items of every XCD y, the longest it
// gives away, XCD after XCD, each in its own order), then the last keep[x] of
// its own items; later slots have no item.  An XCD that gives items away
// receives none, and every XCD's list ends with its own shortest items, which
// fill the last gaps of its CUs.  keep = M and dcnt = 0 everywhere is the
// fixed XCD-major order.  An item is computed the same way on any XCD, so a
// plan changes timing, never results.
constexpr int kXcds = 8;
struct XcdPlan {
  int M;  // items per XCD; 0: no split (item = workgroup index)
  int keep[kXcds], dbeg[kXcds], dcnt[kXcds];
  // Non-zero: the launch is measured; bits 40..63 tag its start stamps.  Every
  // workgroup of a measured launch raises its XCD's end stamp and adds its
  // running time to its XCD's busy time; the first workgroup of each XCD
  // clears both and writes the tagged start stamp (a launch with tag 0 touches
  // none of this).  Stamps: the
  // library's per-GPU array of 3 * 8 values (xcd_stat_address): [x] end,
  // [8 + x] start and [16 + x] busy time of XCD x, in 10 ns ticks of the GPU's
  // constant clock (low 40 bits).
  unsigned long long tag;
};

// The item of workgroup w under plan X, or -1 for a slot without one.
__host__ __device__ inline int64_t xcd_item(const XcdPlan& X, int64_t w) {
  if (X.M == 0) return w;
  const int x = (int)(w % kXcds), sl = (int)(w / kXcds);
  if (sl < X.dcnt[x]) {  // a donated item
    int idx = X.dbeg[x] + sl, y = 0;
    while (y < kXcds - 1 && idx >= X.M - X.keep[y]) {
      idx -= X.M - X.keep[y];
      ++y;
    }
    return (int64_t)y * X.M + idx;
  }
  const int own = sl - X.dcnt[x];
  return own < X.keep[x] ? (int64_t)x * X.M + (X.M - X.keep[x]) + own : -1;
}

// Query block qi and query tile t of the r-th item (r < nqblk * ntq, tiles of
// `rows` rows, blocks of blk rows), longest-first under the causal mask, so
// that the last items an XCD runs are its shortest:
//  * contiguous (block p holds p*blk ..): blocks, then tiles, descending.  The
//    tiles of one block stay together: they walk the key blocks in the same
//    ring order, so the CUs of an XCD that run them at the same time share
//    K/V tiles in its L2.  Non-causal rings of any layout take this order.
//  * striped (block p holds p, p+N, ..): a tile's work depends on its index
//    within the block, not on the block, so tiles descending, and within a
//    tile index blocks descending.  (Blocks first would give every block's
//    list its own long-to-short run, and long items would still start near
//    the end.)
//  * zigzag (block p holds chunk p, then chunk 2N-1-p): the tiles that reach
//    the second chunk, blocks ascending, then the first-chunk tiles, blocks
//    descending, tiles descending within a block; that is longest-first by
//    last query position.
//
// Written without branches: a branch on the layout here changes how the
// compiler allocates the kernel's scalar registers, and the tile loop's walker
// then moves to vector registers.
__host__ __device__ inline void item_tile(int layout, bool causal, int nqblk, int ntq, int rows,
                                          int blk, int r, int& qi, int& t) {
  const int tc = ntq - 1 - r % ntq, qc = nqblk - 1 - r / ntq;    // contiguous
  const int ts = ntq - 1 - r / nqblk, qs = nqblk - 1 - r % nqblk;  // striped
  const int t1 = (blk >> 1) / rows;  // zigzag: tiles wholly inside the first chunk
  const int n2 = ntq - t1;           // and tiles that reach the second chunk
  const bool second = t1 == 0 || r < nqblk * n2;
  const int r1 = r - nqblk * n2, t1d = t1 > 0 ? t1 : 1, n2d = n2 > 0 ? n2 : 1;
  const int tz = second ? ntq - 1 - r % n2d : t1 - 1 - r1 % t1d;
  const int qz = second ? r / n2d : nqblk - 1 - r1 / t1d;
  const bool zz = causal && layout == RA_ZIGZAG;
  const bool sp = causal && layout == RA_STRIPED;
  t = zz ? tz : (sp ? ts : tc);
  qi = zz ? qz : (sp ? qs : qc);
}

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
  int gpl;         // log2 of the query heads of one kv head a workgroup serves
                   // (matrix-core kernel; 0 elsewhere)
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
// Geometry of the matrix-core kernel in a ring launch (state kept on chip)
// over query blocks of `qlen` rows with G = Hq / Hkv query heads per kv head:
// query rows per head in one workgroup, log2 of the heads it serves, and
// resident workgroups per CU.
void mfma_geometry(int D, int qlen, int G, int* rows, int* gpl, int* per_cu);
// Device address, on the current device, of the XCD stamp array (nullptr on
// failure).
void* xcd_stat_address();

// XCD split of a launch of `nwg` workgroups (ra_xcd.hip): fills *X and
// returns the grid size.  `ring`: a whole-ring or one-device ring launch with
// analytic positions, which is split by the device's fixed or measured XCD
// speeds when its mode asks for it (xcd_speeds); any other launch, and every
// launch in the default mode, keeps the fixed XCD-major order.  The plan is
// the kernel's second argument: indexing a field of AttnParams by the XCD
// number would keep the compiler from splitting AttnParams into scalars, and
// the tile loop's walker then moves to vector registers.
int64_t xcd_prepare(const AttnParams& p, int64_t nwg, bool causal, bool ring, int rows,
                    int per_cu, hipStream_t s, XcdPlan* X);
// After a successful launch prepared by xcd_prepare: in measuring mode, read
// its stamps back now and then (stream-ordered, into pinned host memory) to
// update the estimate; otherwise nothing.
void xcd_after_launch(const XcdPlan& X, hipStream_t s);
// The split xcd_prepare would use under per-XCD speeds `speeds` (host only):
// fills *out and returns the grid size, or 0 when the launch is not split.
int64_t xcd_plan_for(const AttnParams& p, int64_t nwg, bool causal, int rows, int per_cu,
                     const float* speeds, XcdPlan* out);
// The current device's XCD split mode and speed estimate.  set = 0: read the
// estimate; returns the mode (0 equal split, 1 fixed speeds, 2 measuring).
// set = 1: split by `speeds` from now on, or equally with speeds NULL (the
// default; launches then touch no host state).  set = 2: measure from equal
// speeds (allocates the read-back on first use).  Returns 0 (set = 1, 2), -1
// without a device, -2 for a speed that is not positive, -3 when the
// read-back cannot be set up.
int xcd_speeds(float* speeds, int* nmeas, int set);
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
// ra_vocab_ce_static: bytes of its per-GPU scratch array, and the array's
// device address on the current device (looked up on the first call on each
// device; nullptr without a device or when the lookup fails).
constexpr int64_t kCeStaticBytes = (int64_t)8 << 20;
void* ce_static_scratch();
hipError_t launch_ce_grad(const void* logits, int64_t ld, const int64_t* target, const float* lse,
                          int64_t N, int64_t V_loc, int64_t start0, int t, float scale, int dtype,
                          void* grad, int64_t ldg, hipStream_t st);
hipError_t launch_out_merge(const void* oa, const float* lsea, const void* ob, const float* lseb,
                            void* oo, float* lseo, int64_t rows, int64_t D, int dtype,
                            hipStream_t s);

}  // namespace ra
