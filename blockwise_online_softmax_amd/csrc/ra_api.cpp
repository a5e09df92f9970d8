// C ABI of libra.so (declared in include/ra.h): argument validation on the
// host, workspace layout and kernel dispatch.  Validation runs before any HIP
// call, so every error path is reachable without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "ra_internal.h"

namespace {

thread_local char g_err[512] = "";

ra_status fail(ra_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

ra_status ok() {
  g_err[0] = '\0';
  return RA_OK;
}

ra_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(RA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return RA_OK;
}

constexpr int64_t kMaxSeq = (int64_t)1 << 31;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
int64_t elem_size(int dtype) { return dtype == RA_BF16 ? 2 : 4; }
bool head_dim_ok(int64_t D) { return D == 8 || D == 16 || D == 32 || D == 64 || D == 128; }
bool layout_ok(int layout) {
  return layout == RA_CONTIGUOUS || layout == RA_STRIPED || layout == RA_ZIGZAG;
}
int64_t round256(int64_t x) { return (x + 255) & ~(int64_t)255; }

ra_status check_dims(const ra_dims* d) {
  if (d == nullptr) return fail(RA_ERR_NULL, "dims is NULL");
  if (d->dtype != RA_F32 && d->dtype != RA_BF16)
    return fail(RA_ERR_DTYPE, "unknown dtype %d", (int)d->dtype);
  if (d->B < 1 || d->Hq < 1 || d->Hkv < 1 || d->Sq < 1 || d->Sk < 1 || d->D < 1)
    return fail(RA_ERR_SHAPE, "all sizes must be >= 1 (B=%lld Hq=%lld Hkv=%lld Sq=%lld Sk=%lld D=%lld)",
                (long long)d->B, (long long)d->Hq, (long long)d->Hkv, (long long)d->Sq,
                (long long)d->Sk, (long long)d->D);
  if (d->Hq % d->Hkv != 0)
    return fail(RA_ERR_SHAPE, "Hq (%lld) must be a multiple of Hkv (%lld)", (long long)d->Hq,
                (long long)d->Hkv);
  if (!head_dim_ok(d->D))
    return fail(RA_ERR_UNSUPPORTED, "head dim %lld not supported (8, 16, 32, 64, 128)",
                (long long)d->D);
  if (d->Sq >= kMaxSeq || d->Sk >= kMaxSeq)
    return fail(RA_ERR_SHAPE, "sequence lengths must be < 2^31");
  if (d->B * d->Hq >= kMaxSeq || d->B * d->Hq * d->Sq >= ((int64_t)1 << 40))
    return fail(RA_ERR_SHAPE, "batch x heads x rows too large");
  if (!(d->scale == d->scale) || isinf(d->scale))
    return fail(RA_ERR_SHAPE, "scale must be finite");
  return RA_OK;
}

float effective_scale(const ra_dims* d) {
  return d->scale > 0.f ? d->scale : (float)(1.0 / sqrt((double)d->D));
}

ra_status check_state(const ra_state* st) {
  if (st == nullptr) return fail(RA_ERR_NULL, "state is NULL");
  if (st->m == nullptr || st->l == nullptr || st->acc == nullptr)
    return fail(RA_ERR_NULL, "state buffers m, l, acc must be non-NULL");
  if (st->B < 1 || st->Hq < 1 || st->Sq < 1 || st->Sq >= kMaxSeq)
    return fail(RA_ERR_SHAPE, "state sizes out of range");
  if (!head_dim_ok(st->D))
    return fail(RA_ERR_UNSUPPORTED, "state head dim %lld not supported", (long long)st->D);
  if (!aligned(st->m, 4) || !aligned(st->l, 4) || !aligned(st->acc, 16))
    return fail(RA_ERR_SHAPE, "state buffers misaligned (acc needs 16 bytes)");
  return RA_OK;
}

ra_status check_ring_args(const ra_dims* d, int N, int layout, int device) {
  ra_status s = check_dims(d);
  if (s != RA_OK) return s;
  if (N < 1) return fail(RA_ERR_SHAPE, "N must be >= 1 (got %d)", N);
  if (!layout_ok(layout)) return fail(RA_ERR_ENUM, "unknown layout %d", layout);
  if (device < -1 || device >= N)
    return fail(RA_ERR_ENUM, "device must be -1 or in [0, N) (got %d, N=%d)", device, N);
  const int64_t S = d->Sk;
  if (S % N != 0) return fail(RA_ERR_SHAPE, "S=%lld not divisible by N=%d", (long long)S, N);
  if (layout == RA_ZIGZAG && S % (2 * (int64_t)N) != 0)
    return fail(RA_ERR_SHAPE, "zigzag needs S %% 2N == 0 (S=%lld N=%d)", (long long)S, N);
  if (device < 0 && d->Sq != S)
    return fail(RA_ERR_SHAPE, "whole ring needs Sq == Sk (Sq=%lld Sk=%lld)", (long long)d->Sq,
                (long long)S);
  if (device >= 0 && d->Sq != S / N)
    return fail(RA_ERR_SHAPE, "device share needs Sq == S/N (Sq=%lld S/N=%lld)",
                (long long)d->Sq, (long long)(S / N));
  return RA_OK;
}

struct WsLayout {
  int64_t q, k, v, out, lse, total;
};

// The matrix-core kernels read and write a whole striped / zigzag ring in
// natural token order (rows addressed through the layout map, 32-bit byte
// offsets from the start of a key/value head, so heads under 4 GiB); the
// vector kernels, and larger heads, run on device-ordered copies in the
// workspace.
bool ring_natural(const ra_dims* d, int layout, int device) {
  return device < 0 && layout != RA_CONTIGUOUS && d->dtype == RA_BF16 &&
         ra::mfma_supports((int)d->D) && d->Sk * d->D * elem_size(d->dtype) < (1LL << 32);
}

WsLayout ring_ws(const ra_dims* d, int layout, int device) {
  WsLayout w = {0, 0, 0, 0, 0, 0};
  if (device >= 0 || layout == RA_CONTIGUOUS || ring_natural(d, layout, device)) return w;
  const int64_t es = elem_size(d->dtype);
  const int64_t S = d->Sk;
  const int64_t qb = round256(d->B * d->Hq * S * d->D * es);
  const int64_t kb = round256(d->B * d->Hkv * S * d->D * es);
  const int64_t lb = round256(d->B * d->Hq * S * 4);
  w.q = 0;
  w.k = w.q + qb;
  w.v = w.k + kb;
  w.out = w.v + kb;
  w.lse = w.out + qb;
  w.total = w.lse + lb;
  return w;
}

ra::AttnParams base_params(const ra_dims* d) {
  ra::AttnParams p;
  memset(&p, 0, sizeof(p));
  p.B = (int)d->B;
  p.Hq = (int)d->Hq;
  p.Hkv = (int)d->Hkv;
  p.scale = effective_scale(d);
  p.sl2 = (float)((double)p.scale * 1.4426950408889634074);
  p.layout = RA_CONTIGUOUS;
  p.N = 1;
  return p;
}

hipError_t launch_attention(const ra::AttnParams& p, int D, int dtype, bool causal, int pos_mode,
                            bool state_io, hipStream_t s, bool natural = false) {
  if (dtype == RA_BF16 && ra::mfma_supports(D))
    return ra::launch_attn_mfma(p, D, causal, pos_mode, state_io, natural, s);
  return ra::launch_attn_valu(p, D, dtype, causal, pos_mode, state_io, s);
}

}  // namespace

extern "C" {

int ra_version(void) { return 105; }

const char* ra_last_error(void) { return g_err; }

ra_status ra_state_init(const ra_state* st, void* stream) {
  ra_status s = check_state(st);
  if (s != RA_OK) return s;
  (void)hipGetLastError();
  s = hip_status(ra::launch_state_init(st->m, st->l, st->acc, st->B * st->Hq * st->Sq, st->D,
                                       (hipStream_t)stream),
                 "ra_state_init launch");
  return s == RA_OK ? ok() : s;
}

ra_status ra_block_step(const void* Q_i, const void* K_j, const void* V_j, const int32_t* q_pos,
                        const int32_t* k_pos, ra_mask mask_mode, const ra_dims* d,
                        const ra_state* st, void* stream) {
  ra_status s = check_dims(d);
  if (s != RA_OK) return s;
  s = check_state(st);
  if (s != RA_OK) return s;
  if (mask_mode != RA_MASK_NONE && mask_mode != RA_MASK_CAUSAL)
    return fail(RA_ERR_ENUM, "unknown mask mode %d", (int)mask_mode);
  if (Q_i == nullptr || K_j == nullptr || V_j == nullptr)
    return fail(RA_ERR_NULL, "Q_i, K_j and V_j must be non-NULL");
  if (mask_mode == RA_MASK_CAUSAL && (q_pos == nullptr || k_pos == nullptr))
    return fail(RA_ERR_NULL, "causal mask needs q_pos and k_pos");
  if (st->B != d->B || st->Hq != d->Hq || st->Sq != d->Sq || st->D != d->D)
    return fail(RA_ERR_SHAPE, "state (B=%lld Hq=%lld Sq=%lld D=%lld) does not match dims",
                (long long)st->B, (long long)st->Hq, (long long)st->Sq, (long long)st->D);
  if (!aligned(Q_i, 16) || !aligned(K_j, 16) || !aligned(V_j, 16))
    return fail(RA_ERR_SHAPE, "Q_i, K_j, V_j must be 16-byte aligned");
  ra::AttnParams p = base_params(d);
  p.Q = Q_i;
  p.K = K_j;
  p.V = V_j;
  p.q_pos = q_pos;
  p.k_pos = k_pos;
  p.m = st->m;
  p.l = st->l;
  p.acc = st->acc;
  p.Sq_tot = d->Sq;
  p.Sk_tot = d->Sk;
  p.nqblk = 1;
  p.qlen = (int)d->Sq;
  p.dev0 = 0;
  p.nkblk = 1;
  p.klen = (int)d->Sk;
  p.blk = (int)d->Sk;
  const bool causal = mask_mode == RA_MASK_CAUSAL;
  (void)hipGetLastError();
  s = hip_status(launch_attention(p, (int)d->D, d->dtype, causal,
                                  causal ? ra::POS_ARRAY : ra::POS_NONE, true, (hipStream_t)stream),
                 "ra_block_step launch");
  return s == RA_OK ? ok() : s;
}

ra_status ra_finalize(const ra_state* st, void* out, float* lse, ra_dtype out_dtype,
                      void* stream) {
  ra_status s = check_state(st);
  if (s != RA_OK) return s;
  if (out == nullptr) return fail(RA_ERR_NULL, "out must be non-NULL");
  if (out_dtype != RA_F32 && out_dtype != RA_BF16)
    return fail(RA_ERR_DTYPE, "unknown out dtype %d", (int)out_dtype);
  if (!aligned(out, out_dtype == RA_BF16 ? 8 : 16) || (lse != nullptr && !aligned(lse, 4)))
    return fail(RA_ERR_SHAPE, "out / lse misaligned");
  (void)hipGetLastError();
  s = hip_status(ra::launch_finalize(st->m, st->l, st->acc, out, lse, st->B * st->Hq * st->Sq,
                                     st->D, out_dtype, (hipStream_t)stream),
                 "ra_finalize launch");
  return s == RA_OK ? ok() : s;
}

// A buffer written by a merge either is the input buffer of the same role
// (in place) or shares no byte with any input buffer or with the other outputs.
struct span {
  const void* p;
  int64_t bytes;
  int role;
};
bool disjoint(const span& x, const span& y) {
  const uintptr_t a = (uintptr_t)x.p, b = (uintptr_t)y.p;
  return a + (uintptr_t)x.bytes <= b || b + (uintptr_t)y.bytes <= a;
}
bool aliasing_ok(const span* outs, int nout, const span* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (!disjoint(outs[i], ins[j]) && !(outs[i].p == ins[j].p && outs[i].role == ins[j].role))
        return false;
    for (int j = 0; j < i; ++j)
      if (!disjoint(outs[i], outs[j])) return false;
  }
  return true;
}

ra_status ra_state_merge(const ra_state* a, const ra_state* b, const ra_state* out,
                         void* stream) {
  ra_status s = check_state(a);
  if (s == RA_OK) s = check_state(b);
  if (s == RA_OK) s = check_state(out);
  if (s != RA_OK) return s;
  for (const ra_state* x : {b, out})
    if (x->B != a->B || x->Hq != a->Hq || x->Sq != a->Sq || x->D != a->D)
      return fail(RA_ERR_SHAPE, "states to merge must have equal B, Hq, Sq, D");
  const int64_t rows = a->B * a->Hq * a->Sq, vb = rows * 4, ab = rows * a->D * 4;
  const span ins[6] = {{a->m, vb, 0}, {a->l, vb, 1}, {a->acc, ab, 2},
                       {b->m, vb, 0}, {b->l, vb, 1}, {b->acc, ab, 2}};
  const span outs[3] = {{out->m, vb, 0}, {out->l, vb, 1}, {out->acc, ab, 2}};
  if (!aliasing_ok(outs, 3, ins, 6))
    return fail(RA_ERR_SHAPE, "ra_state_merge: out overlaps an input other than in place");
  (void)hipGetLastError();
  s = hip_status(ra::launch_state_merge(a->m, a->l, a->acc, b->m, b->l, b->acc, out->m, out->l,
                                        out->acc, rows, a->D,
                                        (hipStream_t)stream),
                 "ra_state_merge launch");
  return s == RA_OK ? ok() : s;
}

ra_status ra_merge(const void* out_a, const float* lse_a, const void* out_b, const float* lse_b,
                   void* out, float* lse, int64_t rows, int64_t D, ra_dtype dtype, void* stream) {
  if (out_a == nullptr || lse_a == nullptr || out_b == nullptr || lse_b == nullptr ||
      out == nullptr || lse == nullptr)
    return fail(RA_ERR_NULL, "ra_merge: every pointer must be non-NULL");
  if (dtype != RA_F32 && dtype != RA_BF16)
    return fail(RA_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  if (rows < 1 || rows >= ((int64_t)1 << 40))
    return fail(RA_ERR_SHAPE, "rows out of range (%lld)", (long long)rows);
  if (!head_dim_ok(D)) return fail(RA_ERR_UNSUPPORTED, "head dim %lld not supported", (long long)D);
  if (!aligned(out_a, 16) || !aligned(out_b, 16) || !aligned(out, 16) || !aligned(lse_a, 4) ||
      !aligned(lse_b, 4) || !aligned(lse, 4))
    return fail(RA_ERR_SHAPE, "ra_merge: buffers misaligned (out 16 bytes, lse 4)");
  const int64_t ob = rows * D * (dtype == RA_BF16 ? 2 : 4), lb = rows * 4;
  const span ins[4] = {{out_a, ob, 0}, {lse_a, lb, 1}, {out_b, ob, 0}, {lse_b, lb, 1}};
  const span outs[2] = {{out, ob, 0}, {lse, lb, 1}};
  if (!aliasing_ok(outs, 2, ins, 4))
    return fail(RA_ERR_SHAPE, "ra_merge: out / lse overlap an input other than in place");
  (void)hipGetLastError();
  ra_status s = hip_status(ra::launch_out_merge(out_a, lse_a, out_b, lse_b, out, lse, rows, D,
                                                dtype, (hipStream_t)stream),
                           "ra_merge launch");
  return s == RA_OK ? ok() : s;
}

namespace {

constexpr int kMaxShards = 1024;

ra_status check_ce_rows(const void* logits, int64_t ld, const int64_t* target, int64_t N,
                        int64_t V_loc, ra_dtype dtype) {
  if (logits == nullptr || target == nullptr)
    return fail(RA_ERR_NULL, "logits and target must be non-NULL");
  if (dtype != RA_F32 && dtype != RA_BF16) return fail(RA_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  if (N < 1 || N >= kMaxSeq) return fail(RA_ERR_SHAPE, "N must be in [1, 2^31)");
  if (V_loc < 1 || V_loc >= ((int64_t)1 << 40)) return fail(RA_ERR_SHAPE, "V_loc out of range");
  if (ld < V_loc) return fail(RA_ERR_SHAPE, "row stride ld must be >= V_loc");
  if (!aligned(logits, dtype == RA_BF16 ? 2 : 4) || !aligned(target, 8))
    return fail(RA_ERR_SHAPE, "logits / target misaligned");
  return RA_OK;
}

struct CeWorkspace {
  int64_t stats, partial, total;  // byte offsets
};
CeWorkspace ce_workspace(int64_t N, int t) {
  CeWorkspace w;
  w.stats = 0;
  w.partial = round256(3 * (int64_t)t * N * 4);
  w.total = w.partial + round256(ra::ce_partial_count(N) * 4);
  return w;
}

}  // namespace

ra_status ra_vocab_ce_shard(const void* logits, int64_t ld, const int64_t* target, int64_t N,
                            int64_t V_loc, int64_t vocab_start, ra_dtype dtype, float* m,
                            float* z_sum, float* pred, void* stream) {
  ra_status s = check_ce_rows(logits, ld, target, N, V_loc, dtype);
  if (s != RA_OK) return s;
  if (m == nullptr || z_sum == nullptr || pred == nullptr)
    return fail(RA_ERR_NULL, "m, z_sum and pred must be non-NULL");
  if (!aligned(m, 4) || !aligned(z_sum, 4) || !aligned(pred, 4))
    return fail(RA_ERR_SHAPE, "m / z_sum / pred misaligned");
  {
    const int64_t es = dtype == RA_BF16 ? 2 : 4;
    const span ins[2] = {{logits, ((N - 1) * ld + V_loc) * es, -1}, {target, N * 8, -2}};
    const span outs[3] = {{m, N * 4, 1}, {z_sum, N * 4, 2}, {pred, N * 4, 3}};
    if (!aliasing_ok(outs, 3, ins, 2))
      return fail(RA_ERR_SHAPE, "m / z_sum / pred overlap each other or an input");
  }
  (void)hipGetLastError();
  s = hip_status(ra::launch_ce_stats(logits, ld, target, N, V_loc, vocab_start, 1, dtype, m, z_sum,
                                     pred, (hipStream_t)stream),
                 "ra_vocab_ce_shard launch");
  return s == RA_OK ? ok() : s;
}

ra_status ra_vocab_ce_combine(const float* m, const float* z_sum, const float* pred, int t,
                              int64_t N, float* loss, float* lse, void* stream) {
  if (m == nullptr || z_sum == nullptr || pred == nullptr || loss == nullptr)
    return fail(RA_ERR_NULL, "m, z_sum, pred and loss must be non-NULL");
  if (t < 1 || t > kMaxShards) return fail(RA_ERR_SHAPE, "t must be in [1, %d]", kMaxShards);
  if (N < 1 || N >= kMaxSeq) return fail(RA_ERR_SHAPE, "N must be in [1, 2^31)");
  if (!aligned(m, 4) || !aligned(z_sum, 4) || !aligned(pred, 4) || !aligned(loss, 4) ||
      (lse != nullptr && !aligned(lse, 4)))
    return fail(RA_ERR_SHAPE, "buffers misaligned");
  {
    const int64_t sb = (int64_t)t * N * 4;
    const span ins[3] = {{m, sb, -1}, {z_sum, sb, -2}, {pred, sb, -3}};
    const span outs[2] = {{loss, N * 4, 1}, {lse, lse != nullptr ? N * 4 : 0, 2}};
    if (!aliasing_ok(outs, 2, ins, 3))
      return fail(RA_ERR_SHAPE, "loss / lse overlap each other or an input");
  }
  (void)hipGetLastError();
  ra_status s = hip_status(ra::launch_ce_combine(m, z_sum, pred, t, N, loss, lse, nullptr, nullptr,
                                                 (hipStream_t)stream),
                           "ra_vocab_ce_combine launch");
  return s == RA_OK ? ok() : s;
}

ra_status ra_vocab_ce_grad(const void* logits, int64_t ld, const int64_t* target, const float* lse,
                           int64_t N, int64_t V_loc, int64_t vocab_start, float scale,
                           ra_dtype dtype, void* grad, int64_t ldg, void* stream) {
  ra_status s = check_ce_rows(logits, ld, target, N, V_loc, dtype);
  if (s != RA_OK) return s;
  if (lse == nullptr || grad == nullptr) return fail(RA_ERR_NULL, "lse and grad must be non-NULL");
  if (ldg < V_loc) return fail(RA_ERR_SHAPE, "row stride ldg must be >= V_loc");
  if (!aligned(lse, 4) || !aligned(grad, dtype == RA_BF16 ? 2 : 4))
    return fail(RA_ERR_SHAPE, "lse / grad misaligned");
  if (!std::isfinite(scale)) return fail(RA_ERR_SHAPE, "scale must be finite");
  const int64_t es = dtype == RA_BF16 ? 2 : 4;
  if (N * ((V_loc * es + 4095) / 4096) >= kMaxSeq)
    return fail(RA_ERR_SHAPE, "N x V_loc too large for one launch (split the rows)");
  const uintptr_t g0 = (uintptr_t)grad, g1 = g0 + (uintptr_t)(((N - 1) * ldg + V_loc) * es);
  const uintptr_t l0 = (uintptr_t)logits, l1 = l0 + (uintptr_t)(((N - 1) * ld + V_loc) * es);
  if (g0 < l1 && l0 < g1) return fail(RA_ERR_SHAPE, "grad overlaps the logits");
  {
    const span ins[2] = {{target, N * 8, -1}, {lse, N * 4, -2}};
    const span outs[1] = {{grad, (int64_t)(g1 - g0), 1}};
    if (!aliasing_ok(outs, 1, ins, 2)) return fail(RA_ERR_SHAPE, "grad overlaps target or lse");
  }
  (void)hipGetLastError();
  s = hip_status(ra::launch_ce_grad(logits, ld, target, lse, N, V_loc, vocab_start, 1, scale,
                                    dtype, grad, ldg, (hipStream_t)stream),
                 "ra_vocab_ce_grad launch");
  return s == RA_OK ? ok() : s;
}

size_t ra_vocab_ce_workspace_bytes(int64_t N, int t) {
  if (N < 1 || N >= kMaxSeq || t < 1 || t > kMaxShards) {
    fail(RA_ERR_SHAPE, "N must be in [1, 2^31) and t in [1, %d]", kMaxShards);
    return (size_t)-1;
  }
  ok();
  return (size_t)ce_workspace(N, t).total;
}

namespace {

// Validation shared by ra_vocab_ce and ra_vocab_ce_static (everything but the
// workspace).
ra_status check_vocab_ce(const void* logits, const int64_t* target, int64_t N, int64_t V, int t,
                         ra_dtype dtype, const float* loss, const float* mean_loss,
                         const float* lse) {
  if (t < 1 || t > kMaxShards) return fail(RA_ERR_SHAPE, "t must be in [1, %d]", kMaxShards);
  if (V < 1 || V % t != 0) return fail(RA_ERR_SHAPE, "V must be a positive multiple of t");
  ra_status s = check_ce_rows(logits, V, target, N, V / t, dtype);
  if (s != RA_OK) return s;
  if (loss == nullptr || mean_loss == nullptr)
    return fail(RA_ERR_NULL, "loss and mean_loss must be non-NULL");
  if (!aligned(loss, 4) || !aligned(mean_loss, 4) || (lse != nullptr && !aligned(lse, 4)))
    return fail(RA_ERR_SHAPE, "loss / mean_loss / lse misaligned");
  return RA_OK;
}

// The shard and combine launches of the whole cross-entropy, with the
// statistics and partial sums in `base` laid out as ce_workspace(N, t) says.
ra_status vocab_ce_launch(const void* logits, const int64_t* target, int64_t N, int64_t V, int t,
                          ra_dtype dtype, float* loss, float* mean_loss, float* lse, char* base,
                          const CeWorkspace& w, void* stream) {
  float* st = reinterpret_cast<float*>(base + w.stats);
  float* partial = reinterpret_cast<float*>(base + w.partial);
  const int64_t V_loc = V / t;
  float* m = st;
  float* zs = st + (int64_t)t * N;
  float* pr = st + 2 * (int64_t)t * N;
  (void)hipGetLastError();
  ra_status s = hip_status(ra::launch_ce_stats(logits, V, target, N, V_loc, 0, t, dtype, m, zs,
                                               pr, (hipStream_t)stream),
                           "ra_vocab_ce shard launch");
  if (s != RA_OK) return s;
  s = hip_status(ra::launch_ce_combine(m, zs, pr, t, N, loss, lse, partial, mean_loss,
                                       (hipStream_t)stream),
                 "ra_vocab_ce combine launch");
  return s == RA_OK ? ok() : s;
}

}  // namespace

ra_status ra_vocab_ce(const void* logits, const int64_t* target, int64_t N, int64_t V, int t,
                      ra_dtype dtype, float* loss, float* mean_loss, float* lse, void* ws,
                      size_t ws_bytes, void* stream) {
  ra_status s = check_vocab_ce(logits, target, N, V, t, dtype, loss, mean_loss, lse);
  if (s != RA_OK) return s;
  const CeWorkspace w = ce_workspace(N, t);
  if (ws == nullptr) return fail(RA_ERR_WORKSPACE, "workspace required (%lld bytes)", (long long)w.total);
  if ((int64_t)ws_bytes < w.total)
    return fail(RA_ERR_WORKSPACE, "workspace too small: %zu < %lld", ws_bytes, (long long)w.total);
  if (!aligned(ws, 256)) return fail(RA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  {
    const int64_t es = dtype == RA_BF16 ? 2 : 4;
    const span ins[3] = {{logits, N * V * es, -1}, {target, N * 8, -2}, {ws, w.total, -3}};
    const span outs[3] = {{loss, N * 4, 1}, {mean_loss, 4, 2}, {lse, lse != nullptr ? N * 4 : 0, 3}};
    if (!aliasing_ok(outs, 3, ins, 3))
      return fail(RA_ERR_SHAPE, "loss / mean_loss / lse overlap each other, an input or the workspace");
  }
  return vocab_ce_launch(logits, target, N, V, t, dtype, loss, mean_loss, lse,
                         static_cast<char*>(ws), w, stream);
}

ra_status ra_vocab_ce_static(const void* logits, const int64_t* target, int64_t N, int64_t V,
                             int t, ra_dtype dtype, float* loss, float* mean_loss, float* lse,
                             void* stream) {
  ra_status s = check_vocab_ce(logits, target, N, V, t, dtype, loss, mean_loss, lse);
  if (s != RA_OK) return s;
  const CeWorkspace w = ce_workspace(N, t);
  if (w.total > ra::kCeStaticBytes)
    return fail(RA_ERR_WORKSPACE,
                "N = %lld rows over t = %d shards need %lld bytes of scratch, more than the "
                "%lld-byte static scratch (ra_vocab_ce with a workspace has no such limit)",
                (long long)N, t, (long long)w.total, (long long)ra::kCeStaticBytes);
  {
    const int64_t es = dtype == RA_BF16 ? 2 : 4;
    const span ins[2] = {{logits, N * V * es, -1}, {target, N * 8, -2}};
    const span outs[3] = {{loss, N * 4, 1}, {mean_loss, 4, 2}, {lse, lse != nullptr ? N * 4 : 0, 3}};
    if (!aliasing_ok(outs, 3, ins, 2))
      return fail(RA_ERR_SHAPE, "loss / mean_loss / lse overlap each other or an input");
  }
  char* base = static_cast<char*>(ra::ce_static_scratch());
  if (base == nullptr)
    return fail(RA_ERR_HIP, "no current HIP device, or the static scratch has no device address");
  return vocab_ce_launch(logits, target, N, V, t, dtype, loss, mean_loss, lse, base, w, stream);
}

size_t ra_ring_workspace_bytes(const ra_dims* d, int N, ra_layout layout, int device) {
  if (check_ring_args(d, N, layout, device) != RA_OK) return (size_t)-1;
  ok();
  return (size_t)ring_ws(d, layout, device).total;
}

// Launch parameters of a ring over N devices (device = -1: all of them).
static ra::AttnParams ring_params(const ra_dims* d, int N, ra_layout layout, int device) {
  const int64_t S = d->Sk;
  const int blk = (int)(S / N);
  ra::AttnParams p = base_params(d);
  p.layout = layout;
  p.N = N;
  p.blk = blk;
  p.nkblk = N;
  p.klen = blk;
  p.Sk_tot = S;
  p.qlen = blk;
  if (device >= 0) {
    p.Sq_tot = blk;
    p.nqblk = 1;
    p.dev0 = device;
  } else {
    p.Sq_tot = S;
    p.nqblk = N;
    p.dev0 = 0;
  }
  return p;
}

ra_status ra_ring(const void* Q, const void* K, const void* V, void* out, float* lse,
                  const ra_dims* d, int N, ra_layout layout, int causal, int device, void* ws,
                  size_t ws_bytes, void* stream) {
  ra_status s = check_ring_args(d, N, layout, device);
  if (s != RA_OK) return s;
  if (causal != 0 && causal != 1) return fail(RA_ERR_ENUM, "causal must be 0 or 1 (got %d)", causal);
  if (Q == nullptr || K == nullptr || V == nullptr || out == nullptr || lse == nullptr)
    return fail(RA_ERR_NULL, "Q, K, V, out and lse must be non-NULL");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(out, 16) ||
      !aligned(lse, 4))
    return fail(RA_ERR_SHAPE, "Q, K, V, out must be 16-byte aligned and lse 4-byte aligned");
  const WsLayout w = ring_ws(d, layout, device);
  if (w.total > 0) {
    if (ws == nullptr) return fail(RA_ERR_WORKSPACE, "workspace of %lld bytes required",
                                   (long long)w.total);
    if ((int64_t)ws_bytes < w.total)
      return fail(RA_ERR_WORKSPACE, "workspace too small: %zu < %lld bytes", ws_bytes,
                  (long long)w.total);
    if (!aligned(ws, 256)) return fail(RA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  const hipStream_t st = (hipStream_t)stream;
  const int64_t S = d->Sk;
  const int blk = (int)(S / N);
  const int64_t es = elem_size(d->dtype);
  const int64_t row_bytes = d->D * es;

  ra::AttnParams p = ring_params(d, N, layout, device);
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.out = out;
  p.lse = lse;

  (void)hipGetLastError();
  char* wsb = (char*)ws;
  const bool permuted = w.total > 0;
  if (permuted) {
    s = hip_status(ra::launch_permute(Q, wsb + w.q, d->B * d->Hq, S, row_bytes, N, layout, 0, st),
                   "permute Q");
    if (s != RA_OK) return s;
    s = hip_status(ra::launch_permute(K, wsb + w.k, d->B * d->Hkv, S, row_bytes, N, layout, 0, st),
                   "permute K");
    if (s != RA_OK) return s;
    s = hip_status(ra::launch_permute(V, wsb + w.v, d->B * d->Hkv, S, row_bytes, N, layout, 0, st),
                   "permute V");
    if (s != RA_OK) return s;
    p.Q = wsb + w.q;
    p.K = wsb + w.k;
    p.V = wsb + w.v;
    p.out = wsb + w.out;
    p.lse = (float*)(wsb + w.lse);
  }
  s = hip_status(launch_attention(p, (int)d->D, d->dtype, causal != 0,
                                  causal ? ra::POS_ANALYTIC : ra::POS_NONE, false, st,
                                  ring_natural(d, layout, device)),
                 "ring attention launch");
  if (s != RA_OK) return s;
  if (permuted) {
    s = hip_status(ra::launch_permute(wsb + w.out, out, d->B * d->Hq, S, row_bytes, N, layout, 1,
                                      st),
                   "un-permute out");
    if (s != RA_OK) return s;
    s = hip_status(ra::launch_permute(wsb + w.lse, lse, d->B * d->Hq, S, 4, N, layout, 1, st),
                   "un-permute lse");
    if (s != RA_OK) return s;
  }
  return ok();
}

ra_status ra_permute(const void* src, void* dst, int64_t outer, int64_t S, int64_t row_bytes,
                     int N, ra_layout layout, int inverse, void* stream) {
  if (src == nullptr || dst == nullptr) return fail(RA_ERR_NULL, "src and dst must be non-NULL");
  if (!layout_ok(layout)) return fail(RA_ERR_ENUM, "unknown layout %d", (int)layout);
  if (inverse != 0 && inverse != 1) return fail(RA_ERR_ENUM, "inverse must be 0 or 1");
  if (outer < 1 || S < 1 || S >= kMaxSeq || N < 1)
    return fail(RA_ERR_SHAPE, "outer, S, N must be >= 1 and S < 2^31");
  if (row_bytes < 4 || row_bytes % 4 != 0)
    return fail(RA_ERR_SHAPE, "row_bytes must be a positive multiple of 4 (got %lld)",
                (long long)row_bytes);
  if (S % N != 0) return fail(RA_ERR_SHAPE, "S=%lld not divisible by N=%d", (long long)S, N);
  if (layout == RA_ZIGZAG && S % (2 * (int64_t)N) != 0)
    return fail(RA_ERR_SHAPE, "zigzag needs S %% 2N == 0");
  const uintptr_t al = row_bytes % 16 == 0 ? 16 : 4;
  if (!aligned(src, al) || !aligned(dst, al)) return fail(RA_ERR_SHAPE, "src / dst misaligned");
  (void)hipGetLastError();
  ra_status s = hip_status(ra::launch_permute(src, dst, outer, S, row_bytes, N, layout, inverse,
                                              (hipStream_t)stream),
                           "ra_permute launch");
  return s == RA_OK ? ok() : s;
}

static ra_status check_layout_args(int64_t S, int N, ra_layout layout, int device) {
  if (!layout_ok(layout)) return fail(RA_ERR_ENUM, "unknown layout %d", (int)layout);
  if (S < 1 || S >= kMaxSeq || N < 1) return fail(RA_ERR_SHAPE, "S, N must be >= 1, S < 2^31");
  if (device < -1 || device >= N) return fail(RA_ERR_ENUM, "device must be -1 or in [0, N)");
  if (S % N != 0) return fail(RA_ERR_SHAPE, "S not divisible by N");
  if (layout == RA_ZIGZAG && S % (2 * (int64_t)N) != 0)
    return fail(RA_ERR_SHAPE, "zigzag needs S %% 2N == 0");
  return RA_OK;
}

int64_t ra_xcd_plan(const ra_dims* d, int N, ra_layout layout, int causal, int device,
                    const float* speeds, int* plan) {
  if (check_ring_args(d, N, layout, device) != RA_OK) return -1;
  if (causal != 0 && causal != 1) {
    fail(RA_ERR_ENUM, "causal must be 0 or 1 (got %d)", causal);
    return -1;
  }
  if (speeds == nullptr || plan == nullptr) {
    fail(RA_ERR_NULL, "speeds and plan must be non-NULL");
    return -1;
  }
  for (int x = 0; x < ra::kXcds; ++x)
    if (!(speeds[x] > 0.f) || speeds[x] > 1e6f) {
      fail(RA_ERR_SHAPE, "speeds must be positive and finite");
      return -1;
    }
  memset(plan, 0, sizeof(int) * (1 + 3 * ra::kXcds));
  ok();
  if (!(d->dtype == RA_BF16 && ra::mfma_supports((int)d->D))) return 0;
  ra::AttnParams p = ring_params(d, N, layout, device);
  int rows, per_cu;
  ra::mfma_geometry((int)d->D, p.qlen, p.Hq / p.Hkv, &rows, &p.gpl, &per_cu);
  p.ntq = (p.qlen + rows - 1) / rows;
  const int64_t nwg = (int64_t)p.B * (p.Hq >> p.gpl) * p.nqblk * p.ntq;
  ra::XcdPlan X;
  const int64_t grid = ra::xcd_plan_for(p, nwg, causal != 0, rows, per_cu, speeds, &X);
  if (grid > 0) {
    plan[0] = X.M;
    for (int x = 0; x < ra::kXcds; ++x) {
      plan[1 + x] = X.keep[x];
      plan[1 + ra::kXcds + x] = X.dbeg[x];
      plan[1 + 2 * ra::kXcds + x] = X.dcnt[x];
    }
  }
  return grid;
}

ra_status ra_xcd_speeds(float* speeds, int* nmeas, int set) {
  if (set < 0 || set > 2) return fail(RA_ERR_ENUM, "set must be 0, 1 or 2 (got %d)", set);
  const int r = ra::xcd_speeds(speeds, nmeas, set);
  if (r == -1) return fail(RA_ERR_HIP, "no current HIP device");
  if (r == -2) return fail(RA_ERR_SHAPE, "speeds must be positive and finite");
  if (r == -3) return fail(RA_ERR_HIP, "could not set up the read-back (pinned memory, event)");
  return ok();
}

int64_t ra_layout_position(int64_t S, int N, ra_layout layout, int device, int64_t index) {
  if (check_layout_args(S, N, layout, device) != RA_OK) return -1;
  const int blk = (int)(S / N);
  if (index < 0 || index >= (device < 0 ? S : blk)) {
    fail(RA_ERR_SHAPE, "index out of range");
    return -1;
  }
  const int p = device < 0 ? (int)(index / blk) : device;
  const int a = device < 0 ? (int)(index - (int64_t)p * blk) : (int)index;
  ok();
  return ra::layout_pos(layout, N, blk, p, a);
}

ra_status ra_positions(int32_t* pos, int64_t S, int N, ra_layout layout, int device,
                       void* stream) {
  if (pos == nullptr) return fail(RA_ERR_NULL, "pos must be non-NULL");
  ra_status c = check_layout_args(S, N, layout, device);
  if (c != RA_OK) return c;
  (void)hipGetLastError();
  ra_status s = hip_status(ra::launch_positions(pos, S, N, layout, device, (hipStream_t)stream),
                           "ra_positions launch");
  return s == RA_OK ? ok() : s;
}

}  // extern "C"
