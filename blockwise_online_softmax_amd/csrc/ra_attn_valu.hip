// Vector-ALU attention step: fp32 inputs (every head dim) and bf16 inputs
// with head dims the matrix-core kernel does not take.  Exact online softmax
// ("Module 23: Distributed Training", "The Math: One Block at a Time"): per
// row a running max m, denominator l and unnormalised output o; each chunk of
// up to 16 keys is folded in with the rescale factor exp(m_old - m_new).
//
// Mapping: one wave = 16 query rows x 4 lanes; each lane keeps D/4 elements
// of its row's q and o in registers, a score is a lane-partial dot product
// reduced over the row's 4 lanes.  Keys and values are read straight from
// global memory (all 16 rows of a wave read the same key: one cache line).
#include "ra_internal.h"

namespace ra {

namespace {

constexpr int kRowsPerWave = 16;
constexpr int kWaves = 4;
constexpr int kRowsPerWG = kRowsPerWave * kWaves;
constexpr int kChunk = 16;

template <typename T>
__device__ inline float ld(const T* p);
template <>
__device__ inline float ld<float>(const float* p) { return *p; }
template <>
__device__ inline float ld<uint16_t>(const uint16_t* p) {
  return __uint_as_float(((unsigned)*p) << 16);
}

template <typename T>
__device__ inline void st(T* p, float v);
template <>
__device__ inline void st<float>(float* p, float v) { *p = v; }
template <>
__device__ inline void st<uint16_t>(uint16_t* p, float v) {
  *reinterpret_cast<__bf16*>(p) = (__bf16)v;  // round to nearest even
}

template <int D, typename T, bool CAUSAL, int POS, bool STATE_IO>
__global__ __launch_bounds__(kRowsPerWG * 4) void attn_valu_kernel(AttnParams P) {
  constexpr int DL = D / 4;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int part = lane & 3;
  const int slot = lane >> 2;

  int64_t L = blockIdx.x;
  const int t = (int)(L % P.ntq);
  L /= P.ntq;
  const int qi = (int)(L % P.nqblk);
  L /= P.nqblk;
  const int h = (int)(L % P.Hq);
  const int b = (int)(L / P.Hq);
  const int G = P.Hq / P.Hkv;
  const int g = h / G;
  const int dev = P.dev0 + qi;

  const int la = t * kRowsPerWG + wave * kRowsPerWave + slot;  // local row in block
  const bool rvalid = la < P.qlen;
  const int64_t qrow = (int64_t)qi * P.qlen + la;
  const int64_t bh = (int64_t)b * P.Hq + h;
  const T* Qp = reinterpret_cast<const T*>(P.Q) + (bh * P.Sq_tot + qrow) * D + part * DL;
  const int64_t kvoff = ((int64_t)b * P.Hkv + g) * P.Sk_tot * D + part * DL;
  const T* Kp = reinterpret_cast<const T*>(P.K) + kvoff;
  const T* Vp = reinterpret_cast<const T*>(P.V) + kvoff;

  float q[DL], o[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) q[e] = rvalid ? ld<T>(Qp + e) : 0.f;

  int qpos = 0;
  if (CAUSAL) {
    if (!rvalid)
      qpos = INT32_MIN;
    else if (POS == POS_ARRAY)
      qpos = P.q_pos[qrow];
    else
      qpos = layout_pos(P.layout, P.N, P.blk, dev, la);
  }

  float m = -__builtin_inff(), l = 0.f;
  const int64_t srow = bh * P.Sq_tot + qrow;
  if (STATE_IO && rvalid) {
    m = P.m[srow];
    l = P.l[srow];
#pragma unroll
    for (int e = 0; e < DL; ++e) o[e] = P.acc[srow * D + part * DL + e];
  } else {
#pragma unroll
    for (int e = 0; e < DL; ++e) o[e] = 0.f;
  }

  // Folds the chunk's first n keys into (m, l, o); kv(kk, e, vsel) gives
  // element e of this lane's part of key kk's row (vsel = 0) or value row
  // (vsel = 1), kp(kk) the key's global position (used when CAUSAL).
  auto fold = [&](int n, auto&& kv, auto&& kp) {
    float sc[kChunk];
    bool any = false;
#pragma unroll
    for (int kk = 0; kk < kChunk; ++kk) {
      const bool valid = kk < n;
      bool vis = valid;
      if (CAUSAL && valid) vis = kp(kk) <= qpos;
      float d = 0.f;
      if (valid) {
#pragma unroll
        for (int e = 0; e < DL; ++e) d = fmaf(q[e], kv(kk, e, 0), d);
      }
      d += __shfl_xor(d, 1);
      d += __shfl_xor(d, 2);
      sc[kk] = vis ? d * P.scale : -__builtin_inff();
      any |= vis;
    }
    if (!__any(any)) return;
    float cmax = -__builtin_inff();
#pragma unroll
    for (int kk = 0; kk < kChunk; ++kk) cmax = fmaxf(cmax, sc[kk]);
    const float mnew = fmaxf(m, cmax);
    if (mnew > -__builtin_inff()) {
      const float alpha = expf(m - mnew);  // m = -inf gives 0
      l *= alpha;
#pragma unroll
      for (int e = 0; e < DL; ++e) o[e] *= alpha;
#pragma unroll
      for (int kk = 0; kk < kChunk; ++kk) {
        // The value rows of every key in range are read whether or not the
        // key is visible (a masked key gets p = 0), so their loads do not
        // wait for the scores and share a memory round trip with the keys.
        if (kk < n) {
          const float p = sc[kk] > -__builtin_inff() ? expf(sc[kk] - mnew) : 0.f;
          l += p;
#pragma unroll
          for (int e = 0; e < DL; ++e) o[e] = fmaf(p, kv(kk, e, 1), o[e]);
        }
      }
      m = mnew;
    }
  };
  auto ring_block = [&](int s) { return ((dev - s) % P.nkblk + P.nkblk) % P.nkblk; };

  if constexpr (DL <= 2) {
    // Head dim 8: a chunk's key and value rows and key positions fit in
    // registers.  Chunks are cut from the ring-ordered key sequence as a whole
    // (block after block, across block boundaries), and the next chunk is read
    // while this one is folded, so short blocks do not each wait for memory.
    const int total = P.nkblk * P.klen;
    float kc[kChunk][DL], vc[kChunk][DL];
    int pc[kChunk];
    auto load = [&](int f0, float (&kd)[kChunk][DL], float (&vd)[kChunk][DL], int (&pd)[kChunk]) {
      // key f0 + kk is index a of ring step sb (block j); one division per
      // chunk, then (a, j) advance key by key
      int sb = f0 / P.klen;
      int a = f0 - sb * P.klen;
      int j = ring_block(sb);
#pragma unroll
      for (int kk = 0; kk < kChunk; ++kk) {
        if (f0 + kk < total) {
          const int64_t r = (int64_t)j * P.klen + a;
#pragma unroll
          for (int e = 0; e < DL; ++e) {
            kd[kk][e] = ld<T>(Kp + r * D + e);
            vd[kk][e] = ld<T>(Vp + r * D + e);
          }
          pd[kk] = !CAUSAL ? 0 : POS == POS_ARRAY ? P.k_pos[r] : layout_pos(P.layout, P.N, P.blk, j, a);
          if (++a == P.klen) {  // next ring step: the block before j
            a = 0;
            j = j == 0 ? P.nkblk - 1 : j - 1;
          }
        }
      }
    };
    load(0, kc, vc, pc);
    for (int f0 = 0; f0 < total; f0 += kChunk) {
      const bool more = f0 + kChunk < total;
      float kn[kChunk][DL], vn[kChunk][DL];
      int pn[kChunk];
      if (more) load(f0 + kChunk, kn, vn, pn);
      fold(min(kChunk, total - f0),
           [&](int kk, int e, int vsel) { return vsel ? vc[kk][e] : kc[kk][e]; },
           [&](int kk) { return pc[kk]; });
      if (!more) break;
#pragma unroll
      for (int kk = 0; kk < kChunk; ++kk) {
        pc[kk] = pn[kk];
#pragma unroll
        for (int e = 0; e < DL; ++e) {
          kc[kk][e] = kn[kk][e];
          vc[kk][e] = vn[kk][e];
        }
      }
    }
  } else {
    for (int s = 0; s < P.nkblk; ++s) {
      const int j = ring_block(s);
      const int64_t kb0 = (int64_t)j * P.klen;
      for (int a0 = 0; a0 < P.klen; a0 += kChunk)
        fold(min(kChunk, P.klen - a0),
             [&](int kk, int e, int vsel) {
               return ld<T>((vsel ? Vp : Kp) + (kb0 + a0 + kk) * D + e);
             },
             [&](int kk) {
               return POS == POS_ARRAY ? P.k_pos[kb0 + a0 + kk]
                                       : layout_pos(P.layout, P.N, P.blk, j, a0 + kk);
             });
    }
  }

  if (!rvalid) return;
  if (STATE_IO) {
    if (part == 0) {
      P.m[srow] = m;
      P.l[srow] = l;
    }
#pragma unroll
    for (int e = 0; e < DL; ++e) P.acc[srow * D + part * DL + e] = o[e];
  } else {
    T* op = reinterpret_cast<T*>(P.out) + srow * D + part * DL;
    const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int e = 0; e < DL; ++e) st<T>(op + e, o[e] * inv);
    if (part == 0) P.lse[srow] = l > 0.f ? m + logf(l) : -__builtin_inff();
  }
}

template <int D, typename T>
hipError_t launch_d(const AttnParams& p0, bool causal, int pos_mode, bool state_io,
                    hipStream_t s) {
  AttnParams p = p0;
  p.ntq = (p.qlen + kRowsPerWG - 1) / kRowsPerWG;
  const int64_t nwg = (int64_t)p.B * p.Hq * p.nqblk * p.ntq;
  const dim3 grid((unsigned)nwg), block(kRowsPerWG * 4);
  if (!causal) {
    if (state_io)
      hipLaunchKernelGGL((attn_valu_kernel<D, T, false, POS_NONE, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((attn_valu_kernel<D, T, false, POS_NONE, false>), grid, block, 0, s, p);
  } else if (pos_mode == POS_ARRAY) {
    if (state_io)
      hipLaunchKernelGGL((attn_valu_kernel<D, T, true, POS_ARRAY, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((attn_valu_kernel<D, T, true, POS_ARRAY, false>), grid, block, 0, s, p);
  } else {
    if (state_io)
      hipLaunchKernelGGL((attn_valu_kernel<D, T, true, POS_ANALYTIC, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((attn_valu_kernel<D, T, true, POS_ANALYTIC, false>), grid, block, 0, s,
                         p);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const AttnParams& p, int D, bool causal, int pos_mode, bool state_io,
                    hipStream_t s) {
  switch (D) {
    case 8: return launch_d<8, T>(p, causal, pos_mode, state_io, s);
    case 16: return launch_d<16, T>(p, causal, pos_mode, state_io, s);
    case 32: return launch_d<32, T>(p, causal, pos_mode, state_io, s);
    case 64: return launch_d<64, T>(p, causal, pos_mode, state_io, s);
    case 128: return launch_d<128, T>(p, causal, pos_mode, state_io, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_valu(const AttnParams& p, int D, int dtype, bool causal, int pos_mode,
                            bool state_io, hipStream_t s) {
  if (dtype == RA_BF16) return launch_t<uint16_t>(p, D, causal, pos_mode, state_io, s);
  return launch_t<float>(p, D, causal, pos_mode, state_io, s);
}

}  // namespace ra
