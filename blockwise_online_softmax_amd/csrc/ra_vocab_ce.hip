// Vocab-parallel cross-entropy ("3.6 Distributed Training II", "Vocab-
// parallel cross-entropy"): the loss of a row of logits z with target id t is
// logsumexp(z) - z[t]; with the vocab split into shards, each shard reduces
// its own columns to a row max, a sum of exponentials and the target logit
// (if it owns the target), and three reductions over the shards combine them.
// Its gradient is softmax(z) - onehot(t), already split like the logits.
//
// The page takes the global row max first and then sums exp(z - max) in a
// second pass over the logits.  Here each shard makes one pass: the row's
// (max, sum) pair is kept online, blockwise, exactly as the attention kernels
// keep (m, l), and the combine step rescales every shard's sum to the global
// max (the order-free merge of partial states).  The logits are read once.
//
// All kernels are HBM-bound.  The statistics kernel gives one 256-thread
// workgroup to each (row, shard); each thread reads 16-byte vectors (8 bf16 or
// 4 fp32 logits), four at a time, takes their max, rescales its running sum
// when the max rises and adds the exponentials (base 2, log2(e) folded into
// one FMA).  Rows whose shard does not start on a 16-byte boundary take their
// first and last few logits one at a time.
#include <mutex>

#include "ra_internal.h"

namespace ra {

namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int kThreads = 256;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegInf = -__builtin_inff();

__device__ inline float bf16_at(const char* p, int64_t j) {
  const unsigned short u = reinterpret_cast<const unsigned short*>(p)[j];
  return __uint_as_float((unsigned)u << 16);  // exact
}
template <bool BF16>
__device__ inline float elem(const char* row, int64_t j) {
  if (BF16) return bf16_at(row, j);
  return reinterpret_cast<const float*>(row)[j];
}
// the 16-byte vector v of a 16-byte aligned run of logits, as floats
template <bool BF16>
__device__ inline void load_vec(const char* base, int64_t v, float* x) {
  const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + v);
  if (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
  }
}

// Running (max, sum of exp(x - max)) pairs.  Empty: (-inf, 0).  Branch
// free: while the max is -inf every value seen is -inf or NaN, and with a
// shift of 0 their exponentials are 0 or NaN, which keeps a NaN visible.
__device__ inline float shift_of(float m) { return m == kNegInf ? 0.f : -m * kLog2e; }
__device__ inline void raise_max(float& m, float& s, float gm) {
  const float mn = fmaxf(m, gm);
  s *= m == kNegInf ? 0.f : __builtin_amdgcn_exp2f((m - mn) * kLog2e);
  m = mn;
}
__device__ inline void add_one(float& m, float& s, float x) {
  raise_max(m, s, x);
  s += __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, shift_of(m)));
}
__device__ inline void merge_pair(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  const float a = m == kNegInf ? s : s * __builtin_amdgcn_exp2f((m - M) * kLog2e);
  const float b = m2 == kNegInf ? s2 : s2 * __builtin_amdgcn_exp2f((m2 - M) * kLog2e);
  m = M;
  s = a + b;  // an empty side's sum is 0 (or a NaN kept visible)
}

// One workgroup per (row r = blockIdx.x, shard k = blockIdx.y); the shard's
// logits start at column k * V_loc of a row (row stride ld elements) and own
// the vocab ids start0 + k * V_loc + [0, V_loc).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void ce_stats_kernel(const void* logits, int64_t ld,
                                                            const int64_t* target, int64_t N,
                                                            int64_t V_loc, int64_t start0,
                                                            float* mo, float* so, float* po) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int VEC = 16 / ES;
  constexpr int U = 2;  // vectors in flight per thread
  const int64_t r = blockIdx.x;
  const int k = blockIdx.y;
  const int tid = threadIdx.x;
  const char* row = reinterpret_cast<const char*>(logits) + (r * ld + (int64_t)k * V_loc) * ES;

  const int64_t mis = (int64_t)((uintptr_t)row & 15) / ES;
  const int64_t head = min(mis ? (int64_t)VEC - mis : (int64_t)0, V_loc);
  const int64_t nvec = (V_loc - head) / VEC;
  const int64_t tail0 = head + nvec * VEC;

  float m = kNegInf, s = 0.f;
  for (int64_t j = tid; j < head; j += kThreads) add_one(m, s, elem<BF16>(row, j));
  for (int64_t j = tail0 + tid; j < V_loc; j += kThreads) add_one(m, s, elem<BF16>(row, j));
  const char* body = row + head * ES;
  for (int64_t v0 = tid; v0 < nvec; v0 += U * kThreads) {
    float x[U][VEC];
    float gm = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + (int64_t)u * kThreads;
      if (v < nvec) {
        load_vec<BF16>(body, v, x[u]);
      } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) x[u][i] = kNegInf;
      }
#pragma unroll
      for (int i = 0; i < VEC; ++i) gm = fmaxf(gm, x[u][i]);
    }
    raise_max(m, s, gm);
    const float ms = shift_of(m);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < VEC; ++i) s += __builtin_amdgcn_exp2f(__builtin_fmaf(x[u][i], kLog2e, ms));
  }

// workgroup reduction of the pairs: within each wave, then across waves
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o);
    const float s2 = __shfl_xor(s, o);
    merge_pair(m, s, m2, s2);
  }
  __shared__ float wm[kThreads / 64], ws[kThreads / 64];
  if ((tid & 63) == 0) {
    wm[tid >> 6] = m;
    ws[tid >> 6] = s;
  }
  __syncthreads();
  if (tid == 0) {
    m = wm[0];
    s = ws[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) merge_pair(m, s, wm[w], ws[w]);
    const int64_t start = start0 + (int64_t)k * V_loc;
    const int64_t tg = target[r];
    const float p = (tg >= start && tg < start + V_loc) ? elem<BF16>(row, tg - start) : 0.f;
    const int64_t o = (int64_t)k * N + r;
    mo[o] = m;
    so[o] = s;
    po[o] = p;
  }
}

// Per row: the three reductions over the t shards, loss and lse; with
// `partial`, each workgroup (one wavefront, so that small N still spreads
// over many CUs) also writes the sum of its rows' losses, in a fixed order,
// for the mean.
constexpr int kCombine = 64;
__global__ __launch_bounds__(kCombine) void ce_combine_kernel(const float* m, const float* s,
                                                              const float* p, int t, int64_t N,
                                                              float* loss, float* lse,
                                                              float* partial) {
  const int64_t r = (int64_t)blockIdx.x * kCombine + threadIdx.x;
  float lv = 0.f;
  if (r < N) {
    float M = kNegInf;
#pragma unroll 4
    for (int k = 0; k < t; ++k) M = fmaxf(M, m[(int64_t)k * N + r]);
    float Z = 0.f, P = 0.f;
#pragma unroll 4
    for (int k = 0; k < t; ++k) {
      const float mk = m[(int64_t)k * N + r];
      const float sk = s[(int64_t)k * N + r];
      Z += mk == kNegInf ? sk : sk * expf(mk - M);  // an empty shard adds its 0 (or NaN)
      P += p[(int64_t)k * N + r];
    }
    const float l = M + logf(Z);  // -inf for a row of -inf logits
    lv = l - P;
    loss[r] = lv;
    if (lse != nullptr) lse[r] = l;
  }
  if (partial == nullptr) return;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) lv += __shfl_xor(lv, o);
  if (threadIdx.x == 0) partial[blockIdx.x] = lv;
}

// mean = (sum of the partial sums, fixed order) / N; one workgroup
__global__ __launch_bounds__(kThreads) void ce_mean_kernel(const float* partial, int64_t nb,
                                                           int64_t N, float* mean) {
  __shared__ float red[kThreads];
  float a = 0.f;
  for (int64_t i = threadIdx.x; i < nb; i += kThreads) a += partial[i];
  red[threadIdx.x] = a;
  __syncthreads();
#pragma unroll
  for (int w = kThreads / 2; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *mean = red[0] / (float)N;
}

__device__ inline unsigned pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

// grad = scale * (exp(z - lse) - onehot); scale * exp2(y) is computed as
// exp2(y + log2|scale|) and the one-hot entry is fixed in the one vector
// that holds it.  VEC16 (both rows start on 16-byte boundaries and hold a
// whole number of vectors): one 16-byte vector per thread, the workgroups of
// a row (blockIdx.x = row * chunks + chunk) covering it in one pass, which
// streams faster than a workgroup looping over its row.  Otherwise one
// workgroup per row, one logit per step.  Shard k = blockIdx.y.
template <bool BF16, bool VEC16>
__global__ __launch_bounds__(kThreads) void ce_grad_kernel(const void* logits, int64_t ld,
                                                           const int64_t* target, const float* lse,
                                                           int64_t V_loc, int64_t start0,
                                                           float scale, void* grad, int64_t ldg,
                                                           int64_t chunks) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int VEC = 16 / ES;
  const int64_t r = VEC16 ? (int64_t)blockIdx.x / chunks : (int64_t)blockIdx.x;
  const int k = blockIdx.y;
  const int tid = threadIdx.x;
  const char* row = reinterpret_cast<const char*>(logits) + (r * ld + (int64_t)k * V_loc) * ES;
  char* grow = reinterpret_cast<char*>(grad) + (r * ldg + (int64_t)k * V_loc) * ES;
  // exp2 shift with |scale| folded in as its log2; the sign applied after
  const float ls = -lse[r] * kLog2e + __builtin_amdgcn_logf(fabsf(scale));
  const float sg = scale < 0.f ? -1.f : 1.f;
  const int64_t tj = target[r] - (start0 + (int64_t)k * V_loc);  // local target column
  if (VEC16) {
    const int64_t v = ((int64_t)blockIdx.x - r * chunks) * kThreads + tid;
    if (v >= V_loc / VEC) return;
    float x[VEC];
    load_vec<BF16>(row, v, x);
    float g[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) g[i] = sg * __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], kLog2e, ls));
    if (tj >= 0 && v == tj / VEC) {
#pragma unroll
      for (int i = 0; i < VEC; ++i)
        if (i == tj % VEC) g[i] -= scale;
    }
    u32x4 w;
    if (BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(g[2 * i], g[2 * i + 1]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(g[i]);
    }
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(grow) + v);
  } else {
    for (int64_t j = tid; j < V_loc; j += kThreads) {
      float g = sg * __builtin_amdgcn_exp2f(__builtin_fmaf(elem<BF16>(row, j), kLog2e, ls));
      if (j == tj) g -= scale;
      if (BF16) {
        f32x2 v = {g, 0.f};
        const unsigned w = __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
        reinterpret_cast<unsigned short*>(grow)[j] = (unsigned short)(w & 0xffffu);
      } else {
        reinterpret_cast<float*>(grow)[j] = g;
      }
    }
  }
}

}  // namespace

hipError_t launch_ce_stats(const void* logits, int64_t ld, const int64_t* target, int64_t N,
                           int64_t V_loc, int64_t start0, int t, int dtype, float* m, float* s,
                           float* p, hipStream_t st) {
  const dim3 g((unsigned)N, (unsigned)t), b(kThreads);
  if (dtype == RA_BF16)
    hipLaunchKernelGGL(ce_stats_kernel<true>, g, b, 0, st, logits, ld, target, N, V_loc, start0, m,
                       s, p);
  else
    hipLaunchKernelGGL(ce_stats_kernel<false>, g, b, 0, st, logits, ld, target, N, V_loc, start0,
                       m, s, p);
  return hipGetLastError();
}

int64_t ce_partial_count(int64_t N) { return (N + kCombine - 1) / kCombine; }

hipError_t launch_ce_combine(const float* m, const float* s, const float* p, int t, int64_t N,
                             float* loss, float* lse, float* partial, float* mean, hipStream_t st) {
  const int64_t nb = ce_partial_count(N);
  hipLaunchKernelGGL(ce_combine_kernel, dim3((unsigned)nb), dim3(kCombine), 0, st, m, s, p, t, N,
                     loss, lse, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || mean == nullptr) return e;
  hipLaunchKernelGGL(ce_mean_kernel, dim3(1), dim3(kThreads), 0, st, partial, nb, N, mean);
  return hipGetLastError();
}

hipError_t launch_ce_grad(const void* logits, int64_t ld, const int64_t* target, const float* lse,
                          int64_t N, int64_t V_loc, int64_t start0, int t, float scale, int dtype,
                          void* grad, int64_t ldg, hipStream_t st) {
  const int es = dtype == RA_BF16 ? 2 : 4;
  const bool vec = ((uintptr_t)logits % 16 == 0) && ((uintptr_t)grad % 16 == 0) &&
                   (ld * es) % 16 == 0 && (ldg * es) % 16 == 0 && (V_loc * es) % 16 == 0;
  const int64_t chunks = (V_loc * es / 16 + kThreads - 1) / kThreads;
  const dim3 gv((unsigned)(N * chunks), (unsigned)t), gs((unsigned)N, (unsigned)t), b(kThreads);
  if (dtype == RA_BF16) {
    if (vec)
      hipLaunchKernelGGL((ce_grad_kernel<true, true>), gv, b, 0, st, logits, ld, target, lse, V_loc,
                         start0, scale, grad, ldg, chunks);
    else
      hipLaunchKernelGGL((ce_grad_kernel<true, false>), gs, b, 0, st, logits, ld, target, lse,
                         V_loc, start0, scale, grad, ldg, chunks);
  } else {
    if (vec)
      hipLaunchKernelGGL((ce_grad_kernel<false, true>), gv, b, 0, st, logits, ld, target, lse,
                         V_loc, start0, scale, grad, ldg, chunks);
    else
      hipLaunchKernelGGL((ce_grad_kernel<false, false>), gs, b, 0, st, logits, ld, target, lse,
                         V_loc, start0, scale, grad, ldg, chunks);
  }
  return hipGetLastError();
}

// Scratch of ra_vocab_ce_static (for callers that cannot allocate): the
// per-shard statistics and the partial sums of the mean, kCeStaticBytes on each
// GPU the library runs on, held until the process ends.  In host code the name
// `scratch` stands for a host-side shadow, not for the GPU's copy: the kernels
// get the device address that hipGetSymbolAddress returns, looked up once per
// device with that device current.
static __device__ __align__(256) char scratch[kCeStaticBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device (nullptr: not looked up)
}  // namespace

void* ce_static_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace ra
