// bf16 attention step on the CDNA4 matrix cores (gfx950).
//
// The method ("Module 23: Distributed Training", "The Math: One Block at a
// Time"; "3.6 Distributed Training II", "Ring Attention"): a query block stays
// resident while key/value blocks stream past; per query row a running max m,
// a denominator l and an unnormalised output o are rescaled by exp(m_old -
// m_new) and updated with each block's exp(s - m_new) and exp(s - m_new) v.
//
// Work split.  A workgroup owns BM = 32*NW query rows of one (batch, query
// head) and walks the key/value blocks in ring order, 64 keys per tile; each
// of its NW waves owns 32 query rows.  Per tile and wave:
//   S^T[64 keys x 32 queries] = K_tile . Q^T   v_mfma_f32_32x32x16_bf16,
//        A = K rows from LDS, B = Q^T fragments held in registers,
//   softmax on S^T: every lane holds 32 scores of ONE query (the other 32 of
//        that query sit in lane ^ 32), so the row max needs one cross-lane
//        exchange and the running state (m, l, o) is per lane,
//   O^T[D x 32 queries] += V^T . P^T   v_mfma_f32_32x32x16_bf16,
//        A = V^T from LDS (V is transposed while it is written to LDS),
//        B = P straight from the S^T accumulators rounded to bf16.  The key
//        order inside the contraction is permuted to match the lane layout of
//        S^T; V^T is read with the same permutation.
// Operands (32x32x16): lane l holds A[l%32][8*(l/32) .. +8] and
// B[8*(l/32) .. +8][l%32]; accumulator element i of lane l is
// C[8*(i/4) + 4*(l/32) + i%4][l%32].
//
// Exponentials run in base 2 with scale*log2(e) folded into one FMA.  The
// reference max used for the exponentials is only raised when the tile max
// exceeds it by more than 2^8 (lazy rescale): the identity holds for any
// reference value, p stays <= 256 (exact range for bf16 and fp32 sums), and
// the 64-wide rescale of o is skipped for most tiles.  The exact running max
// is tracked beside it and applied before the state leaves the kernel.
//
// Causal masking on global positions (key visible iff pos_k <= pos_q).  With
// device-ordered data (POS_ANALYTIC) positions are computed from the layout
// and ascend inside each device block, so whole blocks / tiles past the query
// tile's last position are skipped and tiles wholly before its first
// position run without a mask.  With explicit position arrays (POS_ARRAY)
// every tile is classified from the min/max of its key positions.
//
// K and V tiles are double-buffered in LDS (global -> registers -> LDS, one
// barrier per tile); the next tile's global loads are in flight while the
// current tile is computed.  LDS layouts are XOR-swizzled so that both the
// writes and the MFMA operand reads are free of bank conflicts.
#include "ra_internal.h"

namespace ra {

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int BN = 64;            // keys per tile
constexpr float kLazy = 8.0f;     // log2 of the largest p admitted before rescaling
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

// A key tile to process: keys [start, start + n) of the Sk_tot axis, from key
// block j (local indices a0 .. a0+n-1); `full` = no element needs a mask.
struct Tile {
  int64_t start;
  int j, a0, n;
  bool full;
  int kp;  // POS_ARRAY: this lane's key position (key start + lane), for masking
};

template <int D, int NW, bool CAUSAL, int POS>
struct TileWalker {
  // uniform walk state
  int s, tt, j;
  bool bfull;
  int ntile_blk;

  __device__ void init(const AttnParams& P) {
    s = 0;
    tt = 0;
    j = 0;
    bfull = false;
    ntile_blk = (P.klen + BN - 1) / BN;
  }

  // Advance to the next tile with at least one visible pair.
  __device__ bool next(const AttnParams& P, int dev, int qmin, int qmax, Tile& T) {
    const int lane = threadIdx.x & 63;
    while (s < P.nkblk) {
      if (tt == 0) {
        j = ((dev - s) % P.nkblk + P.nkblk) % P.nkblk;  // ring order
        bfull = !CAUSAL;
        if (CAUSAL && POS == POS_ANALYTIC) {
          const int kf = layout_pos(P.layout, P.N, P.blk, j, 0);
          const int kl = layout_pos(P.layout, P.N, P.blk, j, P.klen - 1);
          if (kf > qmax) {
            ++s;
            continue;
          }
          bfull = kl <= qmin;
        }
      }
      if (tt >= ntile_blk) {
        ++s;
        tt = 0;
        continue;
      }
      const int a0 = tt * BN;
      const int n = min(BN, P.klen - a0);
      T.start = (int64_t)j * P.klen + a0;
      T.j = j;
      T.a0 = a0;
      T.n = n;
      T.kp = 0;
      bool full = (n == BN);
      if (CAUSAL && POS == POS_ANALYTIC && !bfull) {
        const int kf = layout_pos(P.layout, P.N, P.blk, j, a0);
        const int kl = layout_pos(P.layout, P.N, P.blk, j, a0 + n - 1);
        if (kf > qmax) {  // positions ascend in a block: nothing after is visible
          ++s;
          tt = 0;
          continue;
        }
        full = full && (kl <= qmin);
      }
      ++tt;
      if (CAUSAL && POS == POS_ARRAY) {
        const int kp = lane < n ? P.k_pos[T.start + lane] : 0;
        const int kmin = wave_min(lane < n ? kp : INT32_MAX);
        const int kmax = wave_max(lane < n ? kp : INT32_MIN);
        if (kmin > qmax) continue;
        full = full && (kmax <= qmin);
        T.kp = kp;
      }
      T.full = full;
      return true;
    }
    return false;
  }
};

template <int D, int NW, bool CAUSAL, int POS, bool STATE_IO>
__global__ __launch_bounds__(NW * 64, 2) void attn_mfma_kernel(AttnParams P) {
  constexpr int NC = D / 16;     // 16-wide d chunks of the QK^T contraction
  constexpr int NDB = D / 32;    // 32-row d blocks of O^T
  constexpr int UNITS = D / 8;   // 16-byte units per K row
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32;
  constexpr int KUNITS = BN * UNITS;           // 16-byte units per K tile
  constexpr int KPER = (KUNITS + NT - 1) / NT;
  constexpr int VTASKS = (BN / 4) * (D / 8);   // 4 keys x 8 d per task
  constexpr int VPER = (VTASKS + NT - 1) / NT;
  constexpr int KSW = UNITS < 16 ? UNITS - 1 : 15;  // K swizzle mask

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 31;
  const int hi = lane >> 5;

  // ---- work item: XCD-major, then batch / kv head, longest-first tiles ----
  const int64_t W = (int64_t)P.B * P.Hq * P.nqblk * P.ntq;
  const int64_t w = blockIdx.x;
  int64_t L = (W % 8 == 0) ? (w % 8) * (W / 8) + w / 8 : w;
  const int G = P.Hq / P.Hkv;
  const int hg = (int)(L % G);
  L /= G;
  const int t = P.ntq - 1 - (int)(L % P.ntq);
  L /= P.ntq;
  const int qi = P.nqblk - 1 - (int)(L % P.nqblk);
  L /= P.nqblk;
  const int g = (int)(L % P.Hkv);
  const int b = (int)(L / P.Hkv);
  const int h = g * G + hg;
  const int dev = P.dev0 + qi;

  const int a0q = t * BM;                       // first local row of the tile
  const int nrows = min(BM, P.qlen - a0q);
  const int la = a0q + wave * 32 + r;           // this lane's local query row
  const bool rvalid = la < P.qlen;
  const int64_t qrow = (int64_t)qi * P.qlen + la;
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
      qpos = rvalid ? layout_pos(P.layout, P.N, P.blk, dev, la) : INT32_MIN;
      qmin = layout_pos(P.layout, P.N, P.blk, dev, a0q);
      qmax = layout_pos(P.layout, P.N, P.blk, dev, a0q + nrows - 1);
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

  // ---- tile loaders ----
  u32x4 kreg[KPER];
  u32x4 vreg[VPER][4];
  auto gload = [&](const Tile& T) {
#pragma unroll
    for (int e = 0; e < KPER; ++e) {
      const int x = tid + e * NT;
      const int key = x / UNITS, u = x % UNITS;
      kreg[e] = (x < KUNITS && key < T.n)
                    ? *reinterpret_cast<const u32x4*>(Kg + (T.start + key) * D + u * 8)
                    : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int e = 0; e < VPER; ++e) {
      const int y = tid + e * NT;
      const int kq = y % 16, dq = y / 16;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = 4 * kq + rr;
        vreg[e][rr] = (y < VTASKS && key < T.n)
                          ? *reinterpret_cast<const u32x4*>(Vg + (T.start + key) * D + dq * 8)
                          : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int e = 0; e < KPER; ++e) {
      const int x = tid + e * NT;
      if (x < KUNITS) {
        const int key = x / UNITS, u = x % UNITS;
        *reinterpret_cast<u32x4*>(&Ks[buf][key * D + ((u ^ (key & KSW)) * 8)]) = kreg[e];
      }
    }
#pragma unroll
    for (int e = 0; e < VPER; ++e) {
      const int y = tid + e * NT;
      if (y < VTASKS) {
        const int kq = y % 16, dq = y / 16;
        const u32x4 r0 = vreg[e][0], r1 = vreg[e][1], r2 = vreg[e][2], r3 = vreg[e][3];
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
          // d = 8dq + 2wi (low halves) and 8dq + 2wi + 1 (high halves)
          const u32x2 lo = {(r0[wi] & 0xffffu) | (r1[wi] << 16),
                            (r2[wi] & 0xffffu) | (r3[wi] << 16)};
          const u32x2 hv = {(r0[wi] >> 16) | (r1[wi] & 0xffff0000u),
                            (r2[wi] >> 16) | (r3[wi] & 0xffff0000u)};
          const int d0 = dq * 8 + 2 * wi, d1 = d0 + 1;
          *reinterpret_cast<u32x2*>(&Vt[buf][d0 * BN + ((kq ^ (d0 & 15)) * 4)]) = lo;
          *reinterpret_cast<u32x2*>(&Vt[buf][d1 * BN + ((kq ^ (d1 & 15)) * 4)]) = hv;
        }
      }
    }
  };

  TileWalker<D, NW, CAUSAL, POS> walker;
  walker.init(P);
  Tile cur;
  bool have = walker.next(P, dev, qmin, qmax, cur);
  if (have) {
    gload(cur);
    lstore(0);
  }
  __syncthreads();
  int buf = 0;

  while (have) {
    Tile nxt;
    const bool have_next = walker.next(P, dev, qmin, qmax, nxt);
    if (have_next) gload(nxt);

    // ---- S^T = K . Q^T (two 32-key blocks) ----
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key = kb * 32 + r;
        const int u = 2 * c + hi;
        const u32x4 a = *reinterpret_cast<const u32x4*>(&Ks[buf][key * D + ((u ^ (key & KSW)) * 8)]);
        sacc[kb] = mfma(a, qf[c], sacc[kb]);
      }
    }

    // ---- mask (partial tiles only) ----
    if (!cur.full) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kt = kb * 32 + 8 * (i / 4) + 4 * hi + (i % 4);
          bool vis = kt < cur.n;
          if (CAUSAL) {
            int kp;
            if (POS == POS_ANALYTIC)
              kp = layout_pos(P.layout, P.N, P.blk, cur.j, cur.a0 + kt);
            else
              kp = __shfl(cur.kp, kt);
            vis = vis && (kp <= qpos);
          }
          if (!vis) sacc[kb][i] = -__builtin_inff();
        }
    }

    // ---- online softmax (base 2, lazy rescale) ----
    float tmax = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[kb][i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float tm2 = tmax * P.sl2;
    mtrue = fmaxf(mtrue, tm2);
    const bool need = tm2 > m2 + kLazy;
    if (__any(need)) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m2 - tm2) : 1.0f;
      m2 = need ? tm2 : m2;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }
    const float msub = m2 > -__builtin_inff() ? m2 : 0.f;
    u32x4 pf[2][2];  // bf16 P for the four PV contractions (kb, half)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float pv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i], P.sl2, -msub));
        lsum += pv[i];
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        pf[kb][hh] = u32x4{pack2(pv[8 * hh + 0], pv[8 * hh + 1]), pack2(pv[8 * hh + 2], pv[8 * hh + 3]),
                           pack2(pv[8 * hh + 4], pv[8 * hh + 5]), pack2(pv[8 * hh + 6], pv[8 * hh + 7])};
    }

    // ---- O^T += V^T . P^T ----
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int e8 = 8 * kb + 4 * hh + hi;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d = db * 32 + r;
          const uint16_t* row = &Vt[buf][d * BN];
          const u32x2 x0 = *reinterpret_cast<const u32x2*>(row + ((e8 ^ (d & 15)) * 4));
          const u32x2 x1 = *reinterpret_cast<const u32x2*>(row + (((e8 + 2) ^ (d & 15)) * 4));
          o[db] = mfma(u32x4{x0.x, x0.y, x1.x, x1.y}, pf[kb][hh], o[db]);
        }
      }

    if (have_next) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    cur = nxt;
    have = have_next;
  }

  // ---- epilogue ----
  if (mtrue > -__builtin_inff() && mtrue != m2) {  // move to the exact running max
    const float alpha = __builtin_amdgcn_exp2f(m2 - mtrue);
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    m2 = mtrue;
  }
  const float ltot = lsum + __shfl_xor(lsum, 32);
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

template <int D, int NW>
hipError_t launch_d(const AttnParams& p0, bool causal, int pos_mode, bool state_io,
                    hipStream_t s) {
  AttnParams p = p0;
  p.ntq = (p.qlen + NW * 32 - 1) / (NW * 32);
  const int64_t nwg = (int64_t)p.B * p.Hq * p.nqblk * p.ntq;
  const dim3 grid((unsigned)nwg), block(NW * 64);
  if (!causal) {
    if (state_io)
      hipLaunchKernelGGL((attn_mfma_kernel<D, NW, false, POS_NONE, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((attn_mfma_kernel<D, NW, false, POS_NONE, false>), grid, block, 0, s, p);
  } else if (pos_mode == POS_ARRAY) {
    if (state_io)
      hipLaunchKernelGGL((attn_mfma_kernel<D, NW, true, POS_ARRAY, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((attn_mfma_kernel<D, NW, true, POS_ARRAY, false>), grid, block, 0, s, p);
  } else {
    if (state_io)
      hipLaunchKernelGGL((attn_mfma_kernel<D, NW, true, POS_ANALYTIC, true>), grid, block, 0, s,
                         p);
    else
      hipLaunchKernelGGL((attn_mfma_kernel<D, NW, true, POS_ANALYTIC, false>), grid, block, 0, s,
                         p);
  }
  return hipGetLastError();
}

}  // namespace

bool mfma_supports(int D) { return D == 32 || D == 64 || D == 128; }

hipError_t launch_attn_mfma(const AttnParams& p, int D, bool causal, int pos_mode, bool state_io,
                            hipStream_t s) {
  switch (D) {
    case 32: return launch_d<32, 4>(p, causal, pos_mode, state_io, s);
    case 64: return launch_d<64, 4>(p, causal, pos_mode, state_io, s);
    case 128: return launch_d<128, 4>(p, causal, pos_mode, state_io, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ra
