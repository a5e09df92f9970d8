// bf16 attention step on the CDNA4 matrix cores (gfx950).
//
// The method ("Module 23: Distributed Training", "The Math: One Block at a
// Time"; "3.6 Distributed Training II", "Ring Attention"): a query block stays
// resident while key/value blocks stream past; per query row a running max m,
// a denominator l and an unnormalised output o are rescaled by exp(m_old -
// m_new) and updated with each block's exp(s - m_new) and exp(s - m_new) v.
//
// Work split.  A workgroup owns 32*NW (query row, query head) pairs of one
// batch and kv head and walks the key/value blocks in ring order, 64 keys per
// tile; each of its NW waves owns 32 query rows of one head (NW = 8 for head
// dim 128 and query blocks of at least 256 rows: one 512-thread workgroup per
// CU, two waves per SIMD, each key/value tile shared by 256 query rows;
// otherwise NW = 4, two workgroups per CU).  Under grouped-query attention the
// waves are spread over up to NW query heads of the kv head (the largest power
// of two dividing Hq / Hkv), all on the same positions: the causal walk then
// covers a shorter stretch of positions per workgroup.  Per tile and wave:
//   S^T[64 keys x 32 queries] = K_tile . Q^T   v_mfma_f32_32x32x16_bf16,
//        A = K rows read from LDS, B = Q^T fragments held in registers;
//   softmax on S^T: every lane holds 32 scores of ONE query (the other 32 of
//        that query sit in lane ^ 32), so the row max needs one cross-lane
//        exchange and the running state (m, l, o) is per lane;
//   O^T[D x 32 queries] += V^T . P^T   v_mfma_f32_32x32x16_bf16,
//        A = V^T read from the row-major V tile with the LDS transpose read
//        (ds_read_b64_tr_b16), B = P straight from the S^T accumulators
//        rounded to bf16.  The key order inside the contraction follows the
//        lane layout of S^T and the transpose reads use the same order.
// Operands (32x32x16): lane l holds A[l%32][8*(l/32) .. +8] and
// B[8*(l/32) .. +8][l%32]; accumulator element i of lane l is
// C[8*(i/4) + 4*(l/32) + i%4][l%32].
// ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives element
// i%4 of the 8 bytes that lane 4e + i/4 addressed, as its element e.
//
// Tiles move HBM -> LDS without registers (buffer_load ... lds, 16 bytes per
// lane, through a descriptor bounded by the key/value head), double-buffered,
// one barrier per tile; the next tile's copy is in flight while the current
// one is computed.  Both tiles are row-major with
// the 16-byte units of a row XOR-swizzled (K by row, V by 4*(row bits)) so the MFMA
// operand reads are free of bank conflicts; the swizzle is applied by choosing
// which global unit each lane copies.
//
// Exponentials run in base 2 with scale*log2(e) folded into one FMA, against
// a per-row reference m2 instead of the exact running max: the rescaling
// identity holds for any reference, so the reference only has to keep p
// finite and exact in range.  Two modes:
//  * the state leaves the kernel (block step): m2 is raised to the tile max
//    only when that exceeds it by more than 2^8 (lazy rescale, p <= 256);
//    the exact running max is tracked beside it and applied at the end;
//  * only out and lse leave the kernel (whole ring): no row max is taken at
//    all.  The exponentials use m2 as it stands, and a half-tile whose
//    per-lane sum of p exceeds 2^64 (and, for a real row, every half while
//    m2 is still -inf) is redone after raising m2 to the row max, with l and
//    o rescaled.
//    out and lse do not depend on the reference.
// Either way the rescale of o sits behind a wave-uniform branch that is
// rarely taken.
//
// Causal masking on global positions (key visible iff pos_k <= pos_q).  With
// device-ordered data (POS_ANALYTIC) positions are computed from the layout
// and ascend inside each device block, so whole blocks / tiles past the query
// tile's last position are skipped and tiles wholly before its first
// position run without a mask.  With explicit position arrays (POS_ARRAY)
// every tile is classified from the min/max of its key positions.
#include <utility>

#include "ra_internal.h"

namespace ra {

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((address_space(3))) char lds_t;

constexpr int BN = 64;            // keys per tile
constexpr float kLazy = 8.0f;     // log2 of the largest p admitted before rescaling
constexpr float kBig = 64.0f;     // same, for the checked mode (no row max per tile)
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ inline unsigned pack2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

__device__ inline f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ inline u32x4 lds_read128(const lds_t* p) {
  return *(const __attribute__((address_space(3))) u32x4*)p;
}

__device__ inline u32x2 lds_read_tr(const lds_t* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int n = bytes >= 0xFFFFFFFFll ? (int)0xFFFFFFFFu : (int)(uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
__device__ inline void bdma16(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff, lds_t* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           voff, soff, 0, 0);
}
// The FLAT form, global -> LDS at dst + 16*lane (dst uniform), for kernels
// whose scalar registers are too tight for two buffer descriptors.
__device__ inline void dma16(const void* src, lds_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

__device__ inline void wait_dma() {
  // vmcnt(0); expcnt and lgkmcnt left at their maxima (no wait)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Low 40 bits of the GPU's constant-rate (100 MHz) clock; wraps after 3 hours.
__device__ inline unsigned long long stamp40() {
  return (unsigned long long)__builtin_amdgcn_s_memrealtime() & ((1ull << 40) - 1);
}

}  // namespace

// XCD stamps and busy times of the ring launches (see XcdPlan); one copy per GPU.
__device__ unsigned long long g_xcd_stat[3 * kXcds];

namespace {

// The XCD this wave runs on (hardware register XCC_ID, low 4 bits).
__device__ inline int xcc_id() { return (int)(__builtin_amdgcn_s_getreg((15 << 11) | 20) & 7); }

__device__ inline int wave_min(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ inline int wave_max(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1,
// each call inlined (the step sequences below index registers by i).
template <typename F, int... Is>
__device__ __attribute__((always_inline)) inline void static_for_impl(
    F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// A key tile to process: keys [start, start + n) of the Sk_tot axis, from key
// block j (local indices a0 .. a0+n-1); `full` = no element needs a mask.
// POS_ANALYTIC: key kt of the tile has position (kt < split ? p0 : p1) +
// kt * stride (layouts are piecewise linear in the local index).
// POS_ARRAY: kp = this lane's key position (key start + lane).
struct Tile {
  int64_t start;
  int n;
  bool full;
  int p0, p1, split, stride;
  int kp;
};

// LAY: the layout when fixed at compile time (RA_CONTIGUOUS, RA_STRIPED,
// RA_ZIGZAG), or -1 to read it from the parameters.  A fixed layout turns the
// walker's position arithmetic into a few scalar instructions per tile.
// Walks the key tiles of one query tile in ring order.  With analytic
// positions, the tiles of a key block that the query tile sees, and among
// them the ones it sees whole, are found once per block: positions ascend
// inside a block, so both sets are prefixes of the block's tiles, bounded by
// a binary search (tend: first tile whose first key is past the query tile's
// last position; tfull: first tile whose last key is past its first).  Every
// tile is then a few scalar instructions.  With position arrays, each tile is
// classified from the min / max of its keys' positions.
template <bool CAUSAL, int POS, bool NAT, int LAY = -1>
struct TileWalker {
  int s, tt, j;
  int tend, tfull;  // tiles visited / visited whole in the current block
  int ntile_blk;

  __device__ void init(const AttnParams& P) {
    s = 0;
    tt = 0;
    j = 0;
    tend = 0;
    tfull = 0;
    ntile_blk = (P.klen + BN - 1) / BN;
  }

  // Positions of the keys of the tile at local index a0 of block j (the
  // layouts are piecewise linear in the local index).
  __device__ void positions(const AttnParams& P, int lay, int a0, int n, Tile& T) const {
    T.p0 = layout_pos(lay, P.N, P.blk, j, a0);
    T.stride = lay == RA_STRIPED ? P.N : 1;
    T.split = BN;
    T.p1 = T.p0;
    if (lay == RA_ZIGZAG) {
      const int c = P.blk >> 1;
      if (a0 < c && a0 + n > c) {
        T.split = c - a0;
        T.p1 = layout_pos(lay, P.N, P.blk, j, c) - (c - a0);
      }
    }
  }

  // First tile t in [lo, hi) whose key at local index min(t*BN + off,
  // klen - 1) has a position above lim (hi if none).
  __device__ int first_above(const AttnParams& P, int lay, int lo, int hi, int off,
                             int lim) const {
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (layout_pos(lay, P.N, P.blk, j, min(mid * BN + off, P.klen - 1)) > lim)
        hi = mid;
      else
        lo = mid + 1;
    }
    return lo;
  }

  // Advance to the next tile with at least one visible pair.
  __device__ bool next(const AttnParams& P, int dev, int qmin, int qmax, Tile& T) {
    const int lane = threadIdx.x & 63;
    const int lay = LAY >= 0 ? LAY : P.layout;
    constexpr bool ANALYTIC = CAUSAL && POS == POS_ANALYTIC;
    for (;;) {
      if (tt == 0) {  // a new key block
        if (s >= P.nkblk) return false;
        // ring order (uniform; the first-lane read keeps it scalar, as the
        // remainder is computed in vector registers)
        j = __builtin_amdgcn_readfirstlane(((dev - s) % P.nkblk + P.nkblk) % P.nkblk);
        tend = ntile_blk;
        tfull = CAUSAL ? 0 : ntile_blk;
        if (ANALYTIC) {
          tend = first_above(P, lay, 0, ntile_blk, 0, qmax);
          tfull = first_above(P, lay, 0, tend, BN - 1, qmin);
        }
      }
      if (tt >= tend) {
        ++s;
        tt = 0;
        continue;
      }
      const int a0 = tt * BN;
      const int n = min(BN, P.klen - a0);
      T.start = (int64_t)j * P.klen + a0;
      T.n = n;
      T.kp = 0;
      bool full = n == BN && tt < tfull;
      ++tt;
      if (CAUSAL && POS == POS_ARRAY) {
        const int kp = lane < n ? P.k_pos[T.start + lane] : 0;
        const int kmin = wave_min(lane < n ? kp : INT32_MAX);
        const int kmax = wave_max(lane < n ? kp : INT32_MIN);
        if (kmin > qmax) continue;
        full = n == BN && kmax <= qmin;
        T.kp = kp;
      }
      // positions: for natural-order copies and for the analytic mask
      if (NAT || (ANALYTIC && !full)) positions(P, lay, a0, n, T);
      T.full = full;
      return true;
    }
  }
};

template <int D, int NW, bool CAUSAL, int POS, bool STATE_IO, bool NAT = false, int LAY = -1>
__global__ __launch_bounds__(NW * 64, 2) void attn_mfma_kernel(AttnParams P, XcdPlan X) {
  constexpr int NC = D / 16;          // 16-wide d chunks of the QK^T contraction
  constexpr int NDB = D / 32;         // 32-row d blocks of O^T
  constexpr int UNITS = D / 8;        // 16-byte units per row
  constexpr int ROWB = D * 2;         // bytes per row
  constexpr int TILE_BYTES = BN * ROWB;
  constexpr int XPW = TILE_BYTES / 1024 / NW;  // 1 KB copies per wave per tensor
  constexpr int KMASK = (UNITS < 16 ? UNITS : 16) - 1;
  // V tile swizzle: a transpose read serves 32 lanes per cycle, which read 4
  // key rows x 4 units; XOR by 4 * (row bits) spreads them over all banks.
  constexpr auto vswz = [](int row) -> int {
    return UNITS >= 16 ? 4 * (row & 3) : (UNITS == 8 ? 4 * ((row >> 1) & 1) : 0);
  };
  static_assert(XPW * NW * 1024 == TILE_BYTES, "tile must split into 1 KB copies per wave");

  // two buffers of K and V tiles, then 16 bytes: the workgroup's start stamp
  // (placed last, so every tile offset stays the same)
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * 2 * TILE_BYTES + 16];
  lds_t* smem = (lds_t*)smem_raw;  // generic -> LDS address space

  const int lay = LAY >= 0 ? LAY : P.layout;  // the layout (a constant when LAY >= 0)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index, uniform across the wave (kept in a scalar register)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31;
  const int hi = lane >> 5;

  // ---- work item: XCD plan, then batch / kv head, longest-first tiles ----
  const int64_t w = blockIdx.x;
  int64_t L = xcd_item(X, w);
  if (L < 0) return;  // a slot without an item (the whole workgroup)
  unsigned long long* s_t0 = reinterpret_cast<unsigned long long*>(smem_raw + 2 * 2 * TILE_BYTES);
  if (X.tag != 0 && tid == 0) *s_t0 = stamp40();  // measured launches only
  if (X.tag != 0 && w < kXcds && tid == 0) {  // the first workgroup of an XCD
    const int x = xcc_id();
    g_xcd_stat[x] = 0;
    g_xcd_stat[2 * kXcds + x] = 0;
    g_xcd_stat[kXcds + x] = X.tag | stamp40();
  }
  // A workgroup serves 2^gpl query heads of one kv head over the same R query
  // rows, one wave per 32 rows of one head: its heads share every K / V tile,
  // and its rows span 2^gpl times fewer positions than one head over all the
  // waves would, so the causal bounds of its tile walk are that much tighter.
  constexpr int LNW = NW == 8 ? 3 : 2;
  static_assert((1 << LNW) == NW, "4 or 8 waves");
  const int G = P.Hq / P.Hkv;
  const int wl = LNW - P.gpl;     // log2 of the waves per head
  const int R = 32 << wl;         // query rows per head
  const int ngrp = G >> P.gpl;    // workgroups per (kv head, query tile)
  const int hs = (int)(L % ngrp);
  L /= ngrp;
  const int nt = P.nqblk * P.ntq;
  int qi, t;
  item_tile(lay, CAUSAL && POS == POS_ANALYTIC, P.nqblk, P.ntq, R, P.blk, (int)(L % nt), qi, t);
  L /= nt;
  // Integer division has no scalar form, so the decode above may leave its
  // results in vector registers; they are uniform over the workgroup, and
  // reading the first lane keeps every position and bound derived from them
  // (the walker's included) in scalar registers.
  const int g = __builtin_amdgcn_readfirstlane((int)(L % P.Hkv));
  const int b = __builtin_amdgcn_readfirstlane((int)(L / P.Hkv));
  qi = __builtin_amdgcn_readfirstlane(qi);
  t = __builtin_amdgcn_readfirstlane(t);
  const int h = g * G + (__builtin_amdgcn_readfirstlane(hs) << P.gpl) + (wave >> wl);
  const int dev = P.dev0 + qi;

  const int a0q = t * R;                        // first local row of the tile
  const int nrows = min(R, P.qlen - a0q);
  const int la = a0q + (wave & ((1 << wl) - 1)) * 32 + r;  // this lane's local query row
  const bool rvalid = la < P.qlen;
  // the query row in Q / out / lse: device order, or (NAT) the row's natural
  // token position
  int64_t qrow;
  if constexpr (NAT)
    qrow = rvalid ? layout_pos(lay, P.N, P.blk, dev, la) : 0;
  else
    qrow = (int64_t)qi * P.qlen + la;
  const int64_t bh = (int64_t)b * P.Hq + h;
  const uint16_t* Qg = reinterpret_cast<const uint16_t*>(P.Q);
  const uint16_t* Kg =
      reinterpret_cast<const uint16_t*>(P.K) + ((int64_t)b * P.Hkv + g) * P.Sk_tot * D;
  const uint16_t* Vg =
      reinterpret_cast<const uint16_t*>(P.V) + ((int64_t)b * P.Hkv + g) * P.Sk_tot * D;

  // ---- Q^T fragments (B operand): lane holds Q[row r][16c + 8hi .. +8] ----
  u32x4 qf[NC];
  {
    const uint16_t* qp = Qg + (bh * P.Sq_tot + qrow) * D + hi * 8;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qf[c] = rvalid ? *reinterpret_cast<const u32x4*>(qp + c * 16) : u32x4{0, 0, 0, 0};
  }

  // ---- query positions: this lane's row and the tile's min / max ----
  int qpos = 0, qmin = 0, qmax = 0;
  if (CAUSAL) {
    if (POS == POS_ANALYTIC) {
      qpos = rvalid ? layout_pos(lay, P.N, P.blk, dev, la) : INT32_MIN;
      qmin = layout_pos(lay, P.N, P.blk, dev, a0q);
      qmax = layout_pos(lay, P.N, P.blk, dev, a0q + nrows - 1);
    } else {
      qpos = rvalid ? P.q_pos[qrow] : INT32_MIN;
      int mn = INT32_MAX, mx = INT32_MIN;
      for (int x = lane; x < nrows; x += 64) {
        const int v = P.q_pos[(int64_t)qi * P.qlen + a0q + x];
        mn = min(mn, v);
        mx = max(mx, v);
      }
      qmin = wave_min(mn);
      qmax = wave_max(mx);
    }
  }

  // ---- running state: o (O^T accumulators), m2 (base-2 reference max),
  //      mtrue (exact base-2 running max), lsum (this lane's partial sum) ----
  f32x16 o[NDB];
  float m2 = -__builtin_inff(), mtrue = -__builtin_inff(), lsum = 0.f;
  // Checked mode (the state does not leave the kernel, so only out and lse,
  // which do not depend on the reference, are produced): the exponentials use
  // the current reference m2 directly and no row max is taken; a half whose
  // per-lane sum exceeds plim (p possibly above 2^kBig) is redone after
  // raising m2 to the row max.  While m2 is still -inf, every half of a real
  // row is redone (plim = -1): its visible scores may all be so negative that
  // exp2 underflows to 0, and a zero sum must not pass for "nothing visible".
  // A redo that finds no visible key leaves m2 at -inf.  Padding rows (past
  // the query block) admit a zero sum, so their masked halves are not redone.
  const float plim0 = rvalid ? -1.f : 0.f;  // plim while m2 = -inf
  float msub = 0.f;    // reference subtracted in the exponentials (0 while m2 = -inf)
  float plim = plim0;  // largest admitted per-lane sum of a half
  const int64_t srow = bh * P.Sq_tot + qrow;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  if (STATE_IO && rvalid) {
    const float mv = P.m[srow];
    m2 = mv * kLog2e;
    mtrue = m2;
    lsum = hi == 0 ? P.l[srow] : 0.f;
    const float* ap = P.acc + srow * D + 4 * hi;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(ap + db * 32 + gq * 8);
        o[db][4 * gq + 0] = v.x;
        o[db][4 * gq + 1] = v.y;
        o[db][4 * gq + 2] = v.z;
        o[db][4 * gq + 3] = v.w;
      }
  }

  // ---- per-lane LDS offsets of the MFMA operands (fixed for every tile).
  // The swizzle is a XOR of 16-byte unit indices and the unit index of chunk
  // c (K) or d block db (V) only adds bits above the lane's own, so every
  // offset is the lane's first offset XOR a constant. ----
  // K: row kb*32 + r, unit 2c + hi        -> kofs0 ^ (c << 5)
  const int kofs0 = r * ROWB + ((hi ^ (r & KMASK)) << 4);
  // V^T (transpose reads): key 4hi + (lane%16)/4, d 32db + 16((lane/16)%2) + 4(lane%4)
  //                                       -> vofs0 ^ (db << 6)
  int vofs0;
  {
    const int vkey = 4 * hi + ((lane & 15) >> 2);
    const int u = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    vofs0 = vkey * ROWB + ((u ^ vswz(vkey)) << 4) + ((lane & 1) << 3);
  }

  // ---- tile copy: HBM -> LDS, swizzled.  Copy x = wave + NW*i moves 64
  //      units of 16 bytes: rows x*RPC + lane/UNITS, unit lane%UNITS.  Both
  //      swizzles only depend on row bits that copy i = 0 already fixes
  //      (NW*RPC rows later the pattern repeats), so a full tile's source
  //      offsets are this lane's offset for i = 0 plus i*NW*1024: a uniform
  //      base and a 32-bit lane offset per copy.  Rows past a ragged tile's
  //      end are clamped to its last row. ----
  constexpr int RPC = 64 / UNITS;  // rows per 1 KB copy
  static_assert((NW * RPC) % (KMASK + 1) == 0 && (NW * RPC) % 4 == 0,
                "swizzle period must divide the rows between a wave's copies");
  unsigned dk0, dv0;
  {
    const int row = wave * RPC + lane / UNITS;
    const int ph = lane % UNITS;
    dk0 = row * ROWB + ((ph ^ (row & KMASK)) << 4);
    dv0 = row * ROWB + ((ph ^ vswz(row)) << 4);
  }
  // natural-order rows (NAT): token stride between a tile's rows (N striped,
  // else 1), this lane's source offsets within a copy, and the byte step
  // between a wave's copies
  [[maybe_unused]] unsigned dkn = 0, dvn = 0;
  [[maybe_unused]] int64_t cstep = 0;
  if constexpr (NAT) {
    const int nstride = lay == RA_STRIPED ? P.N : 1;
    const int row = wave * RPC + lane / UNITS;
    const int ph = lane % UNITS;
    dkn = (unsigned)(row * nstride * ROWB) + ((ph ^ (row & KMASK)) << 4);
    dvn = (unsigned)(row * nstride * ROWB) + ((ph ^ vswz(row)) << 4);
    cstep = (int64_t)NW * RPC * nstride * ROWB;
  }
  // One 16-byte-per-lane copy: base + soff is the tile's uniform source and
  // voff the lane's offset.  The 4-wave head-dim-128 kernels have no scalar
  // registers to spare for the two descriptors and use the FLAT form, with the
  // lane offset kept opaque so the address stays "scalar base + 32-bit
  // offset" (the 64-bit-address form of the copy stalls the MFMAs around it).
  constexpr bool kBufCopy = !(D == 128 && NW == 4);
  auto copy16 = [&](const char* base, __amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff,
                    lds_t* dst) {
    if constexpr (kBufCopy) {
      bdma16(r, voff, soff, dst);
    } else {
      unsigned o = voff;
      asm volatile("" : "+v"(o));
      dma16(base + soff + o, dst);
    }
  };
  auto issue_tile = [&](const Tile& T, lds_t* kdst) {
    lds_t* vdst = kdst + TILE_BYTES;
    if constexpr (NAT) {
      // Key rows in natural order: tile row kt is token (kt < split ? p0 : p1)
      // + kt * stride.  The LDS placement (and its swizzle) is the same as
      // for device-ordered rows; only the source rows differ.
      const char* kn = reinterpret_cast<const char*>(Kg);
      const char* vn = reinterpret_cast<const char*>(Vg);
      const int64_t head = P.Sk_tot * ROWB;
      if (T.n == BN && T.split >= BN) {
        // The tile's fields are wave-uniform, but the compiler may hold them
        // in vector registers (zigzag positions are a select between two
        // chunk formulas); reading the first lane keeps the descriptor base
        // scalar, so the copies need no per-lane descriptor loop.
        const int64_t t0 = (int64_t)__builtin_amdgcn_readfirstlane(T.p0) * ROWB;
        const auto kr = rsrc(kn + t0, head - t0), vr = rsrc(vn + t0, head - t0);
#pragma unroll
        for (int i = 0; i < XPW; ++i) {
          const int x = wave + NW * i;
          copy16(kn + t0, kr, dkn, (unsigned)(i * cstep), kdst + x * 1024);
          copy16(vn + t0, vr, dvn, (unsigned)(i * cstep), vdst + x * 1024);
        }
      } else {
        const auto kr = rsrc(kn, head), vr = rsrc(vn, head);
        const int p0 = T.p0, p1 = T.p1, split = T.split, stride = T.stride, last = T.n - 1;
#pragma unroll
        for (int i = 0; i < XPW; ++i) {
          const int x = wave + NW * i;
          const int row = x * RPC + lane / UNITS;
          const int ph = lane % UNITS;
          const int rr = min(row, last);
          const int first = rr < split ? p0 : p1;  // per-lane choice between two uniform values
          const int64_t tok = (int64_t)first + (int64_t)rr * stride;
          unsigned ko = (unsigned)(tok * ROWB) + ((ph ^ (row & KMASK)) << 4);
          unsigned vo = (unsigned)(tok * ROWB) + ((ph ^ vswz(row)) << 4);
          copy16(kn, kr, ko, 0u, kdst + x * 1024);
          copy16(vn, vr, vo, 0u, vdst + x * 1024);
        }
      }
      return;
    }
    const char* kb = reinterpret_cast<const char*>(Kg + T.start * D);
    const char* vb = reinterpret_cast<const char*>(Vg + T.start * D);
    const int64_t rem = (P.Sk_tot - T.start) * ROWB;
    const auto kr = rsrc(kb, rem), vr = rsrc(vb, rem);
    if (T.n == BN) {
#pragma unroll
      for (int i = 0; i < XPW; ++i) {
        const int x = wave + NW * i;
        copy16(kb, kr, dk0, (unsigned)(i * NW * 1024), kdst + x * 1024);
        copy16(vb, vr, dv0, (unsigned)(i * NW * 1024), vdst + x * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < XPW; ++i) {
        const int x = wave + NW * i;
        const int row = x * RPC + lane / UNITS;
        const int ph = lane % UNITS;
        const int rb = min(row, T.n - 1) * ROWB;
        unsigned ko = rb + ((ph ^ (row & KMASK)) << 4), vo = rb + ((ph ^ vswz(row)) << 4);
        copy16(kb, kr, ko, 0u, kdst + x * 1024);
        copy16(vb, vr, vo, 0u, vdst + x * 1024);
      }
    }
  };

  TileWalker<CAUSAL, POS, NAT, LAY> walker;
  walker.init(P);
  Tile cur;
  bool have = walker.next(P, dev, qmin, qmax, cur);
  if (have) issue_tile(cur, smem);
  wait_dma();
  __syncthreads();

  // Causal / ragged mask of one 32-key half (partial tiles only).  The rare
  // branches of the tile (mask, redo, rescale) are marked unlikely, so their
  // code is laid out away from the straight-line path.
  auto mask_half = [&](f32x16& sa, int kb, const Tile& T) {
    if (CAUSAL && POS == POS_ANALYTIC && T.n == BN && T.split >= BN) {
      // Full tile with one linear position map (the common case): key kt is
      // visible iff p0 + kt * stride <= qpos.  With kt = c + 4 hi, c the same
      // in every lane, that is c * stride <= lim: one compare per element.
      const int lim = rvalid ? qpos - T.p0 - 4 * hi * T.stride : INT32_MIN;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = kb * 32 + 8 * (i / 4) + (i % 4);
        sa[i] = c * T.stride <= lim ? sa[i] : -__builtin_inff();
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kt = kb * 32 + 8 * (i / 4) + 4 * hi + (i % 4);
      bool vis = kt < T.n;
      if (CAUSAL) {
        int kp;
        if (POS == POS_ANALYTIC)
          kp = (kt < T.split ? T.p0 : T.p1) + kt * T.stride;
        else
          kp = __shfl(T.kp, kt);
        vis = vis & (kp <= qpos);
      }
      sa[i] = vis ? sa[i] : -__builtin_inff();
    }
  };

  // ---- online softmax of one 32-key half, split so that its pieces can be
  //      placed between MFMAs (base 2, lazy rescale) ----
  // Part 1 (row max and the rescale decision): updates m2 and mtrue and
  // returns the reference subtracted in the exponentials, the previous
  // reference and whether any lane of the wave raised its reference.
  struct Ref {
    float msub, mold;
    bool any;
  };
  auto softmax_max = [&](const f32x16& sa) {
    float tmax = fmaxf(fmaxf(sa[0], sa[1]), sa[2]);
#pragma unroll
    for (int i = 3; i < 16; ++i) tmax = fmaxf(tmax, sa[i]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax),
                                                       false, false);
      tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));  // max over lane and lane^32
    }
    const float tm2 = tmax * P.sl2;
    mtrue = fmaxf(mtrue, tm2);
    const bool need = tm2 > m2 + kLazy;
    Ref R;
    R.mold = m2;
    m2 = need ? tm2 : m2;
    R.any = __any(need);
    R.msub = m2 > -__builtin_inff() ? m2 : 0.f;
    return R;
  };
  // Part 2: exponentials of elements [e0, e1) of the half into pv, summed into ps.
  auto softmax_exp = [&](const f32x16& sa, float msub, float* pv, float& ps, float& psb, int e0,
                         int e1) {
#pragma unroll
    for (int e = e0; e < e1; ++e)
      pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[e], P.sl2, -msub));
#pragma unroll
    for (int e = e0; e < e1; ++e) (e & 1 ? psb : ps) += pv[e];
  };
  auto pack_half = [&](const float* pv, u32x4& pf0, u32x4& pf1) {
    pf0 = u32x4{pack2(pv[0], pv[1]), pack2(pv[2], pv[3]), pack2(pv[4], pv[5]), pack2(pv[6], pv[7])};
    pf1 = u32x4{pack2(pv[8], pv[9]), pack2(pv[10], pv[11]), pack2(pv[12], pv[13]),
                pack2(pv[14], pv[15])};
  };
  // Part 3, once the half's sum is known: rescale l and o when the wave
  // raised a reference (rare under the lazy rule, so the factor and the
  // multiplications sit behind a wave-uniform branch), then add the sum.
  auto softmax_close = [&](const Ref& R, float ps) {
    if (__builtin_expect(R.any, 0)) {
      // 1 where this lane kept its reference (also when both are -inf)
      const float alpha = R.mold == m2 ? 1.0f : __builtin_amdgcn_exp2f(R.mold - m2);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }
    lsum += ps;
  };

  // Checked mode, end of a half: if a lane's sum is out of range (or NaN),
  // the wave takes the pair max, raises m2 where it is exceeded, redoes the
  // half's exponentials and rescales l and o; then the sum joins l.
  auto softmax_check = [&](const f32x16& sa, float* pv, float& ps) {
    if (__builtin_expect(__any(!(ps <= plim)), 0)) {
      float tmax = sa[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, sa[i]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax),
                                                       false, false);
      tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      const float tm2 = tmax * P.sl2;
      const bool raise = tm2 > m2;
      const float mnew = raise ? tm2 : m2;
      const float alpha = raise ? __builtin_amdgcn_exp2f(m2 - mnew) : 1.0f;
      m2 = mnew;
      msub = m2 > -__builtin_inff() ? m2 : 0.f;
      plim = m2 > -__builtin_inff() ? __builtin_amdgcn_exp2f(kBig) : plim0;
      ps = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[e], P.sl2, -msub));
        ps += pv[e];
      }
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }
    lsum += ps;
  };

  // Keeps a softmax result in the region where it is written (an empty asm
  // that reads it), so the compiler cannot sink the exponentials below the
  // branches that follow and lose their overlap with the MFMAs.
  auto pin = [](const u32x4& a, const u32x4& c, float x) {
    asm volatile("" ::"v"(a), "v"(c), "v"(x));
  };

  // One tile: copy the next tile into `nb` while computing on `cb`.  The two
  // restrict-qualified buffers tell the compiler the copy cannot alias the
  // operand reads, so no wait for the copy is placed before them.
  // The tile is one sequence of MFMA steps per wave:
  //   S0 = K[0:32] . Q^T            | next tile's copy issue
  //   S1 = K[32:64] . Q^T           | softmax(S0) in pieces
  //   O^T += V[0:32]^T . P0^T       | softmax(S1) in pieces
  //   O^T += V[32:64]^T . P1^T
  // and the LDS operand of step s + PD is read at step s, across the section
  // boundaries (MFMA and VALU of one wave overlap in hardware; the fences
  // keep the compiler from reordering across the steps).
  constexpr int PD = 3;  // operand read distance, in MFMAs
  // Step at which the next tile's copy is issued.  Ring kernels issue it at
  // the start of the P.V steps, away from the operand reads at the tile's
  // start; half a tile is enough for it to land (a quarter is not).  The
  // later issue also keeps the workgroups of an XCD that stream the same K /
  // V in step: a workgroup that runs ahead of the others is the first to
  // miss in L2 and waits a little at its tile's end, the others then find
  // those tiles in L2.  (Issued halfway through the first QK^T section, the
  // latency was hidden, the 32 workgroups of an XCD drifted apart over a
  // 1M-token device share, and it fetched 0.7-0.9 TB per launch instead of
  // 139 GB.)  The state-in-HBM steps (few tiles per workgroup, each first
  // read from memory) keep the early issue.
  constexpr int kCopyStep = !STATE_IO ? 2 * NC : NC / 2;
  auto tile = [&](const lds_t* __restrict__ cb, lds_t* __restrict__ nb, const Tile& ct,
                  const Tile& nt, bool have_next) {
    const lds_t* Kb = cb;
    const lds_t* Vb = cb + TILE_BYTES;
    constexpr int NSTEP = 2 * NDB;           // (half, d block) PV steps per 32 keys
    constexpr int NS = 2 * NC + 2 * NSTEP;   // MFMAs per tile and wave
    auto operand = [&](int st) -> u32x4 {
      if (st < 2 * NC) {  // K rows 32*kb .. +32, d chunk c
        const int kb = st / NC, c = st % NC;
        return lds_read128(Kb + (kofs0 ^ (c << 5)) + kb * 32 * ROWB);
      }
      const int v = st - 2 * NC;  // V^T: key half kb, 16-key group hh, d block db
      const int kb = v / NSTEP, hh = (v % NSTEP) / NDB, db = v % NDB;
      const lds_t* vp = Vb + (vofs0 ^ (db << 6)) + (32 * kb + 16 * hh) * ROWB;
      const u32x2 x0 = lds_read_tr(vp);
      const u32x2 x1 = lds_read_tr(vp + 8 * ROWB);
      return u32x4{x0.x, x0.y, x1.x, x1.y};
    };

    f32x16 s0, s1;
    u32x4 pf[2][2];
    Ref R0, R1;
    float pv0[16], pv1[16];
    float ps0 = 0.f, ps1 = 0.f, ps0b = 0.f, ps1b = 0.f;
    u32x4 opd[PD + 1];
    static_for<PD>([&](auto I) __attribute__((always_inline)) {
      constexpr int st = decltype(I)::value;
      opd[st] = operand(st);
    });
    static_for<NS>([&](auto I) __attribute__((always_inline)) {
      constexpr int st = decltype(I)::value;
      // Issue priority: raised while the wave's softmax runs beside its
      // MFMAs (sections 2 and 3), normal in the MFMA-only sections (1 and 4):
      // where the two waves of a SIMD compete, the one with vector work
      // pending issues first.
      if constexpr (st == 0 || st == 2 * NC + NSTEP) __builtin_amdgcn_s_setprio(0);
      if constexpr (st == NC) __builtin_amdgcn_s_setprio(1);
      if constexpr (st + PD < NS) opd[(st + PD) % (PD + 1)] = operand(st + PD);
      __builtin_amdgcn_sched_barrier(0);
      const u32x4 a = opd[st % (PD + 1)];
      if constexpr (st < NC) {
        s0 = mfma(a, qf[st], st == 0 ? f32x16{} : s0);
      } else if constexpr (st < 2 * NC) {
        constexpr int c = st - NC;
        s1 = mfma(a, qf[c], c == 0 ? f32x16{} : s1);
        // softmax(S0): the max after the first MFMA (S0's last result has
        // landed by then), the exponentials spread over the rest
        if constexpr (c == 0) {
          if constexpr (STATE_IO) R0 = softmax_max(s0);
        }
        if constexpr (c >= 1)
          softmax_exp(s0, STATE_IO ? R0.msub : msub, pv0, ps0, ps0b, 16 * (c - 1) / (NC - 1),
                      16 * c / (NC - 1));
      } else if constexpr (st < 2 * NC + NSTEP) {
        constexpr int v = st - 2 * NC, hh = v / NDB, db = v % NDB;
        o[db] = mfma(a, pf[0][hh], o[db]);
        if constexpr (v == 0) {
          if constexpr (STATE_IO) R1 = softmax_max(s1);
        }
        if constexpr (v >= 1)
          softmax_exp(s1, STATE_IO ? R1.msub : msub, pv1, ps1, ps1b, 16 * (v - 1) / (NSTEP - 1),
                      16 * v / (NSTEP - 1));
      } else {
        constexpr int v = st - 2 * NC - NSTEP, hh = v / NDB, db = v % NDB;
        o[db] = mfma(a, pf[1][hh], o[db]);
        // Ring kernels: the second P register of half 1 (elements 8..15) is
        // packed here, beside the MFMAs that only use the first one, rather
        // than between the two P.V sections (the empty asm keeps each pack
        // in its step).
        if constexpr (!STATE_IO && v < NDB) {
#pragma unroll
          for (int j = 4 + v * 4 / NDB; j < 4 + (v + 1) * 4 / NDB; ++j) {
            unsigned pk = pack2(pv1[2 * j], pv1[2 * j + 1]);
            asm volatile("" : "+v"(pk));
            pf[1][1][j - 4] = pk;
          }
        }
      }
      if constexpr (st == kCopyStep) issue_tile(have_next ? nt : ct, nb);  // last tile re-copies itself
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (st == NC - 1) {
        if (__builtin_expect(!ct.full, 0)) mask_half(s0, 0, ct);
      } else if constexpr (st == 2 * NC - 1) {
        if constexpr (STATE_IO) {
          pack_half(pv0, pf[0][0], pf[0][1]);
          ps0 += ps0b;
          pin(pf[0][0], pf[0][1], ps0);
          softmax_close(R0, ps0);
        } else {
          ps0 += ps0b;
          softmax_check(s0, pv0, ps0);
          pack_half(pv0, pf[0][0], pf[0][1]);
        }
        if (__builtin_expect(!ct.full, 0)) mask_half(s1, 1, ct);
      } else if constexpr (st == 2 * NC + NSTEP - 1) {
        if constexpr (STATE_IO) {
          pack_half(pv1, pf[1][0], pf[1][1]);
          ps1 += ps1b;
          pin(pf[1][0], pf[1][1], ps1);
          softmax_close(R1, ps1);
        } else {
          ps1 += ps1b;
          softmax_check(s1, pv1, ps1);
          pf[1][0] = u32x4{pack2(pv1[0], pv1[1]), pack2(pv1[2], pv1[3]), pack2(pv1[4], pv1[5]),
                           pack2(pv1[6], pv1[7])};
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // The loop body is written out once per LDS buffer, so that every operand
  // read and copy destination has a constant buffer offset.
  while (have) {
    {
      Tile nxt;
      const bool have_next = walker.next(P, dev, qmin, qmax, nxt);
      tile(smem, smem + 2 * TILE_BYTES, cur, nxt, have_next);
      wait_dma();
      __syncthreads();
      cur = nxt;
      if (!have_next) break;
    }
    {
      Tile nxt;
      const bool have_next = walker.next(P, dev, qmin, qmax, nxt);
      tile(smem + 2 * TILE_BYTES, smem, cur, nxt, have_next);
      wait_dma();
      __syncthreads();
      cur = nxt;
      have = have_next;
    }
  }

  // measured launches: raise the XCD's end stamp, add this workgroup's time
  if (X.tag != 0 && tid == 0) {
    const unsigned long long t1 = stamp40();
    const int x = xcc_id();
    atomicMax(&g_xcd_stat[x], t1);
    atomicAdd(&g_xcd_stat[2 * kXcds + x], (t1 - *s_t0) & ((1ull << 40) - 1));
  }

  // ---- epilogue ----
  if (STATE_IO && mtrue > -__builtin_inff() && mtrue != m2) {  // move to the exact running max
    const float alpha = __builtin_amdgcn_exp2f(m2 - mtrue);
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    m2 = mtrue;
  }
  float ltot;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum),
                                                     false, false);
    ltot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // lane + lane^32
  }
  if (!rvalid) return;
  if (STATE_IO) {
    if (hi == 0) {
      P.m[srow] = m2 * kLn2;
      P.l[srow] = ltot;
    }
    float* ap = P.acc + srow * D + 4 * hi;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
        *reinterpret_cast<f32x4*>(ap + db * 32 + gq * 8) =
            f32x4{o[db][4 * gq], o[db][4 * gq + 1], o[db][4 * gq + 2], o[db][4 * gq + 3]};
  } else {
    const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
    uint16_t* op = reinterpret_cast<uint16_t*>(P.out) + srow * D + 4 * hi;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
        *reinterpret_cast<u32x2*>(op + db * 32 + gq * 8) =
            u32x2{pack2(o[db][4 * gq] * inv, o[db][4 * gq + 1] * inv),
                  pack2(o[db][4 * gq + 2] * inv, o[db][4 * gq + 3] * inv)};
    if (hi == 0)
      P.lse[srow] = ltot > 0.f ? (m2 + __log2f(ltot)) * kLn2 : -__builtin_inff();
  }
}

// log2 of the query heads a workgroup of `nw` waves serves: the largest power
// of two that divides the group size G = Hq / Hkv, at most nw.
int heads_log2(int G, int nw) {
  int l = 0;
  while ((2 << l) <= nw && G % (2 << l) == 0) ++l;
  return l;
}

template <int D, int NW>
hipError_t launch_d(const AttnParams& p0, bool causal, int pos_mode, bool state_io, bool natural,
                    hipStream_t s) {
  AttnParams p = p0;
  p.gpl = heads_log2(p.Hq / p.Hkv, NW);
  const int rows = (NW * 32) >> p.gpl, per_cu = NW == 8 ? 1 : 2;  // rows per head
  p.ntq = (p.qlen + rows - 1) / rows;
  const int64_t nwg = (int64_t)p.B * (p.Hq >> p.gpl) * p.nqblk * p.ntq;
  const bool ring = !state_io && pos_mode != POS_ARRAY;
  XcdPlan X;
  const int64_t ngrid = xcd_prepare(p, nwg, causal, ring, rows, per_cu, s, &X);
  const dim3 grid((unsigned)ngrid), block(NW * 64);
  hipError_t e;
  if (natural) {  // whole ring read and written in natural token order
    if (state_io || pos_mode == POS_ARRAY) return hipErrorInvalidValue;
    if (causal && p.layout == RA_STRIPED)
      hipLaunchKernelGGL((attn_mfma_kernel<D, NW, true, POS_ANALYTIC, false, true, RA_STRIPED>),
                         grid, block, 0, s, p, X);
    else if (causal && p.layout == RA_ZIGZAG)
      hipLaunchKernelGGL((attn_mfma_kernel<D, NW, true, POS_ANALYTIC, false, true, RA_ZIGZAG>),
                         grid, block, 0, s, p, X);
    else if (causal)  // natural order is only for striped and zigzag rings
      return hipErrorInvalidValue;
    else
      hipLaunchKernelGGL((attn_mfma_kernel<D, NW, false, POS_NONE, false, true>), grid, block, 0,
                         s, p, X);
    e = hipGetLastError();
    if (e == hipSuccess) xcd_after_launch(X, s);
    return e;
  }
  if (state_io) {
    // the state-in-HBM steps run 4-wave workgroups only: two share a CU, so
    // one's state loads and stores overlap the other's matrix work
    if constexpr (NW == 8) {
      return hipErrorInvalidValue;
    } else {
      if (!causal)
        hipLaunchKernelGGL((attn_mfma_kernel<D, NW, false, POS_NONE, true>), grid, block, 0, s, p,
                           X);
      else if (pos_mode == POS_ARRAY)
        hipLaunchKernelGGL((attn_mfma_kernel<D, NW, true, POS_ARRAY, true>), grid, block, 0, s, p,
                           X);
      else  // the state-in-HBM steps take explicit positions
        return hipErrorInvalidValue;
    }
  } else if (!causal) {
    hipLaunchKernelGGL((attn_mfma_kernel<D, NW, false, POS_NONE, false>), grid, block, 0, s, p, X);
  } else if (pos_mode == POS_ARRAY) {
    hipLaunchKernelGGL((attn_mfma_kernel<D, NW, true, POS_ARRAY, false>), grid, block, 0, s, p, X);
  } else {
    if (p.layout == RA_CONTIGUOUS)  // ring launches: the layout fixed at compile time
      hipLaunchKernelGGL((attn_mfma_kernel<D, NW, true, POS_ANALYTIC, false, false, RA_CONTIGUOUS>),
                         grid, block, 0, s, p, X);
    else if (p.layout == RA_STRIPED)
      hipLaunchKernelGGL((attn_mfma_kernel<D, NW, true, POS_ANALYTIC, false, false, RA_STRIPED>),
                         grid, block, 0, s, p, X);
    else
      hipLaunchKernelGGL((attn_mfma_kernel<D, NW, true, POS_ANALYTIC, false, false, RA_ZIGZAG>),
                         grid, block, 0, s, p, X);
  }
  e = hipGetLastError();
  if (e == hipSuccess) xcd_after_launch(X, s);
  return e;
}

}  // namespace

bool mfma_supports(int D) { return D == 32 || D == 64 || D == 128; }

void* xcd_stat_address() {
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_xcd_stat)) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return p;
}

void mfma_geometry(int D, int qlen, int G, int* rows, int* gpl, int* per_cu) {
  const int nw = (D == 128 && qlen >= 256) ? 8 : 4;
  *gpl = heads_log2(G, nw);
  *rows = (nw * 32) >> *gpl;
  *per_cu = nw == 8 ? 1 : 2;  // one 8-wave or two 4-wave workgroups share a CU
}

hipError_t launch_attn_mfma(const AttnParams& p, int D, bool causal, int pos_mode, bool state_io,
                            bool natural, hipStream_t s) {
  switch (D) {
    case 32: return launch_d<32, 4>(p, causal, pos_mode, state_io, natural, s);
    case 64: return launch_d<64, 4>(p, causal, pos_mode, state_io, natural, s);
    case 128:  // 8 waves (256 query rows) once a ring block has that many rows
      return (p.qlen >= 256 && !state_io)
                 ? launch_d<128, 8>(p, causal, pos_mode, state_io, natural, s)
                 : launch_d<128, 4>(p, causal, pos_mode, state_io, natural, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ra
