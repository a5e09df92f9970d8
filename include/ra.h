/*
 * ra.h -- C ABI of the MI355X (gfx950) ring-attention library, libra.so.
 *
 * One device's share of ring (sequence-parallel) attention, and a whole ring
 * simulated on one GPU.  A resident query block keeps, per query row, a
 * running max m, a running denominator l and an unnormalised output acc; each
 * key/value block that arrives is folded in with exponential rescaling, and
 * after the last block out = acc / l.  The operation and its notation follow
 *   "Module 23: Distributed Training", sections "Sequence Parallelism: Ring
 *   Attention" and "The Math: One Block at a Time" (the fold and the final
 *   division), "Exact by Construction" (causal ring = causally masked full
 *   attention), "The Causal Imbalance -- and the Striped Fix" (layouts);
 *   "Explain ring attention and how it enables very long contexts across
 *   multiple devices?", section "The ring" (split / compute / pass / repeat
 *   and divide, and the rotation order);
 *   "3.6 Distributed Training II: Tensor, Pipeline, Sequence & Expert
 *   Parallelism", section "Ring Attention" (per-step loop on a device) and
 *   "Vocab-parallel cross-entropy" (log-sum-exp = m + log Z).
 *
 * Conventions shared by every call
 *   - Every tensor and workspace is device memory owned by the caller.  The
 *     library never allocates device memory, and never frees or keeps a
 *     caller's pointer after a call returns.  Its only state is the per-device
 *     XCD split of ra_ring, which by default is the equal split and holds
 *     nothing; measuring it (ra_xcd_speeds) uses a 192-byte array per GPU in
 *     the library's own module and, set up by that call, 192 bytes of pinned
 *     host memory and an event.
 *   - Tensors are dense and row-major with the head dim innermost:
 *       Q, out      [B, Hq,  Sq, D]      K, V   [B, Hkv, Sk, D]
 *       m, l, lse   [B, Hq,  Sq]  fp32   acc    [B, Hq,  Sq, D] fp32
 *     Q, K, V (and out, unless stated) share one element type (ra_dtype).
 *     Device pointers must be 16-byte aligned.
 *   - Query head h reads key/value head h / (Hq / Hkv) (contiguous groups).
 *   - Scores are s = (q . k) * scale; scale <= 0 selects 1/sqrt(D).
 *   - Causal masking is on global token positions: key j is visible to
 *     query i iff pos(j) <= pos(i) (the diagonal is visible).
 *   - `stream` is a hipStream_t (NULL = the null stream), passed as void* so
 *     that this header needs no HIP header and stays plain C.  Calls are
 *     asynchronous on it; none synchronises the device.
 *   - Every argument is validated on the host before anything is launched;
 *     on error nothing is launched, the call returns a non-zero ra_status and
 *     ra_last_error() describes the problem.  No exception crosses the ABI.
 *   - Supported head dims: D in {8, 16, 32, 64, 128}.  bf16 with D in
 *     {32, 64, 128} runs on the matrix cores (bf16 MFMA, fp32 accumulate);
 *     other cases run on a vector-ALU kernel.  Sequence lengths < 2^31.
 */
#ifndef RA_H
#define RA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums are int-sized.  Compiled as C++ they get int32_t as their fixed
 * underlying type: a C caller may pass any int where an enum is expected, and
 * the implementation validates it, which is only well defined in C++ when the
 * enum can hold every int32_t value. */
#ifdef __cplusplus
#define RA_ENUM_BASE : int32_t
#else
#define RA_ENUM_BASE
#endif

typedef enum ra_status RA_ENUM_BASE {
  RA_OK = 0,
  RA_ERR_NULL = 1,        /* a required pointer is NULL                      */
  RA_ERR_SHAPE = 2,       /* sizes inconsistent, not divisible, misaligned   */
  RA_ERR_DTYPE = 3,       /* unknown element type                            */
  RA_ERR_ENUM = 4,        /* unknown mask / layout value, bad device index   */
  RA_ERR_UNSUPPORTED = 5, /* valid but not built (head dim)                  */
  RA_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required      */
  RA_ERR_HIP = 7          /* the HIP runtime reported an error on launch     */
} ra_status;

typedef enum ra_dtype RA_ENUM_BASE { RA_F32 = 0, RA_BF16 = 1 } ra_dtype;
typedef enum ra_mask RA_ENUM_BASE { RA_MASK_NONE = 0, RA_MASK_CAUSAL = 1 } ra_mask;

/* Token -> device layouts of a sequence of S tokens over N devices
 * (blk = S/N tokens each; local index a = 0..blk-1, ascending positions):
 *   RA_CONTIGUOUS  device p holds block p:        pos = p*blk + a
 *   RA_STRIPED     device p holds p, p+N, ...:    pos = p + a*N
 *   RA_ZIGZAG      2N chunks of c = S/(2N); device p holds chunk p and then
 *                  chunk 2N-1-p:  a < c: pos = p*c + a,
 *                                 a >= c: pos = (2N-1-p)*c + (a-c)
 *                  (needs S % 2N == 0).
 * "Device order" concatenates the N device blocks, device 0 first. */
typedef enum ra_layout RA_ENUM_BASE { RA_CONTIGUOUS = 0, RA_STRIPED = 1, RA_ZIGZAG = 2 } ra_layout;

typedef struct ra_dims {
  int64_t B, Hq, Hkv; /* batch, query heads, key/value heads (Hq % Hkv == 0) */
  int64_t Sq, Sk;     /* query rows and key rows per (batch, head)           */
  int64_t D;          /* head dim                                            */
  int32_t dtype;      /* ra_dtype of Q, K, V                                 */
  float scale;        /* score scale; <= 0 means 1/sqrt(D)                   */
} ra_dims;

/* Running state of a query block (fp32, caller-owned device buffers).
 * m[r] is the running max of the scaled scores seen by row r, l[r] the sum of
 * exp(s - m[r]) over them and acc[r, :] the sum of exp(s - m[r]) * v.  A row
 * that has seen no visible key has m = -inf, l = 0, acc = 0. */
typedef struct ra_state {
  float* m;   /* [B, Hq, Sq]    */
  float* l;   /* [B, Hq, Sq]    */
  float* acc; /* [B, Hq, Sq, D] */
  int64_t B, Hq, Sq, D;
} ra_state;

/* The empty state: m = -inf, l = 0, acc = 0.  ("Explain ring attention...",
 * "The ring": the running max starts at -inf, sum and output at zero.) */
ra_status ra_state_init(const ra_state* st, void* stream);

/* Non-finite inputs.  The kernels compute each tile of keys as a whole: a
 * masked key inside a tile that also holds visible keys enters the P.V
 * product with weight exactly 0, so its value row must be finite (0 * inf is
 * NaN).  Keys in tiles or blocks with no visible pair are never read. */

/* Fold one key/value block into the state in place ("Module 23", "The Math:
 * One Block at a Time"): for each row, m' = max(m, max_j s_ij),
 * l = l*e^(m-m') + sum_j e^(s_ij-m'), acc = acc*e^(m-m') + sum_j e^(s_ij-m') v_j.
 *   Q_i [B,Hq,Sq,D], K_j / V_j [B,Hkv,Sk,D] of d->dtype; d describes them and
 *   must match st (B, Hq, Sq, D).
 *   q_pos [Sq], k_pos [Sk]: int32 global positions (shared over batch and
 *   heads); read only for RA_MASK_CAUSAL, may be NULL for RA_MASK_NONE.
 *   Masked pairs contribute nothing; a row with no visible key in this block
 *   keeps its state.  The stored m is the exact running max. */
ra_status ra_block_step(const void* Q_i, const void* K_j, const void* V_j,
                        const int32_t* q_pos, const int32_t* k_pos, ra_mask mask_mode,
                        const ra_dims* d, const ra_state* st, void* stream);

/* out = acc / l in out_dtype (round to nearest even for bf16) and
 * lse = m + ln l in fp32 ("Module 23", "The Math": divide at the end;
 * "3.6 ...", "Vocab-parallel cross-entropy": logsumexp = m + log Z).
 * A row with l == 0 gets out = 0 and lse = -inf.  lse may be NULL. */
ra_status ra_finalize(const ra_state* st, void* out, float* lse, ra_dtype out_dtype,
                      void* stream);

/* The whole ring ("Explain ring attention...", "The ring"): the sequence is
 * split over N virtual devices by `layout`; each device keeps its query block
 * and folds in the N key/value blocks in ring order -- at step s device p
 * holds block (p - s) mod N -- then divides by l.  Blocks (and tiles) with no
 * visible pair are skipped.  Outputs: out (Q's dtype) and lse (fp32).
 *   device == -1: the whole ring on this GPU.  Q, K, V, out, lse are in
 *     natural token order; d->Sq == d->Sk == S.  Under striped and zigzag
 *     layouts, bf16 inputs with head dim 32, 64 or 128 are read and written in
 *     place through the layout map; other inputs (fp32, head dim 8 or 16) are
 *     permuted into device order in the workspace and back afterwards.
 *   device == p (0 <= p < N): device p's share.  Q is p's block in its local
 *     order (d->Sq == S/N), K and V are the whole sequence in device order
 *     (d->Sk == S), and out / lse come back in p's local order.
 *   causal: 0 or 1.  S % N == 0 (S % 2N == 0 for zigzag).
 *   ws / ws_bytes: workspace of at least ra_ring_workspace_bytes(...) bytes
 *   (0 for contiguous layouts, for device >= 0 and for bf16 with head dim 32,
 *   64 or 128; ws may then be NULL). */
ra_status ra_ring(const void* Q, const void* K, const void* V, void* out, float* lse,
                  const ra_dims* d, int N, ra_layout layout, int causal, int device,
                  void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes ra_ring needs for these arguments; (size_t)-1 on invalid
 * arguments (ra_last_error() says why). */
size_t ra_ring_workspace_bytes(const ra_dims* d, int N, ra_layout layout, int device);

/* Layout permutation of rows ("Module 23", "The Causal Imbalance -- and the
 * Striped Fix"): src and dst are [outer, S, row_bytes] byte arrays.  Rows are
 * opaque bytes, so one call moves Q/K/V/out rows (D elements) and lse rows
 * (one fp32) alike.
 *   inverse == 0: natural -> device order, dst[o][p*blk + a] = src[o][pos(p, a)]
 *   inverse == 1: device -> natural order, dst[o][pos(p, a)] = src[o][p*blk + a]
 * row_bytes must be a positive multiple of 4 (16 or more runs vectorised).
 * src and dst must not overlap. */
ra_status ra_permute(const void* src, void* dst, int64_t outer, int64_t S, int64_t row_bytes,
                     int N, ra_layout layout, int inverse, void* stream);

/* int32 global positions, the operands of the causal mask ("Module 23",
 * "Exact by Construction": key visible iff its position is not after the
 * query's; "The Causal Imbalance -- and the Striped Fix": the layouts).
 * device == -1: pos[i] for every index i of a device-ordered sequence
 * (S entries).  device == p: p's block in its local order (S/N entries). */
ra_status ra_positions(int32_t* pos, int64_t S, int N, ra_layout layout, int device,
                       void* stream);

/* The global token position of one index, computed on the host with the same
 * layout map the kernels use ("Module 23", "The Causal Imbalance -- and the
 * Striped Fix"): device == -1: index i of the device-ordered sequence
 * (S entries); device == p: index i of p's block in its local order (S/N
 * entries).  Returns -1 (and sets ra_last_error) on invalid arguments, the
 * same checks as ra_positions. */
int64_t ra_layout_position(int64_t S, int N, ra_layout layout, int device, int64_t index);

/* ---- Work split over the XCDs (not from the pages: a property of the GPU).
 * An MI355X runs a launch on 8 XCDs (dies with their own L2); workgroup w goes
 * to XCD w % 8.  The bf16 matrix-core ring kernel (ra_ring, D 32/64/128)
 * numbers its work items XCD-major, longest first, and by default gives each
 * XCD an equal share; ra_ring then keeps no host state, takes no lock and
 * enqueues nothing but the kernel.  The XCDs of one GPU run a few percent
 * apart, so a caller may ask for a split by per-XCD speeds, given or measured
 * (ra_xcd_speeds): a slow XCD then hands the first (longest) items of its
 * list to faster ones, which run them first, when a simulation of the
 * schedule says the launch ends sooner.  Results are the same bit for bit under any split. */

/* The split ra_ring would use for this ring under per-XCD speeds speeds[8]
 * (relative, any positive scale).  Host only.  plan receives 25 ints: M (items
 * per XCD; XCD x owns items x*M .. x*M+M-1, longest first), keep[8], dbeg[8]
 * and dcnt[8].  XCD x, slot by slot, first runs entries dbeg .. dbeg+dcnt-1 of
 * the donated list (the first M - keep items of every XCD, XCD after XCD),
 * then its own last keep items; slot w / 8 of XCD w % 8 is workgroup w.
 * Returns the grid size in workgroups (8*M with keep = M and dcnt = 0 for the
 * equal split); 0, with plan zeroed, for a launch that is never split (fewer
 * than 64 items per XCD, or not the matrix-core kernel); -1 (and sets
 * ra_last_error) on invalid arguments, the same checks as ra_ring. */
int64_t ra_xcd_plan(const ra_dims* d, int N, ra_layout layout, int causal, int device,
                    const float* speeds, int* plan);

/* The current device's XCD split.
 *   set == 0: copy the speed estimate (mean 1) to speeds[8] and the number of
 *     measurements folded in to *nmeas (either may be NULL).
 *   set == 1: with speeds[8] (relative, positive and finite), split ra_ring
 *     launches on this device by those speeds from now on; with speeds NULL,
 *     split equally (the default).
 *   set == 2: measure the speeds from equal ones on.  This call allocates, once
 *     per device, 192 bytes of pinned host memory and an event (kept until the
 *     process ends).  Each later ring launch of at least 64 items per XCD on
 *     this device records when every XCD starts and ends and how long its
 *     workgroups ran (a 192-byte library array on the GPU); the first 64 such
 *     launches, then one in 8, copy that array on the caller's stream into the
 *     pinned memory, which a later call reads once the copy has landed.
 *     Launches of 1 ms or more count.  A launch inside a stream capture is
 *     split by the current estimate and measures nothing.  Freeze the result
 *     with set == 1 to stop measuring.
 * RA_ERR_HIP without a current device or when the read-back cannot be set up,
 * RA_ERR_SHAPE for a speed that is not positive and finite, RA_ERR_ENUM for
 * another value of set. */
ra_status ra_xcd_speeds(float* speeds, int* nmeas, int set);

/* Merge two states of the same rows built from disjoint key sets into `out`
 * ("Module 23", "The Math: One Block at a Time": the fold does not depend on
 * the order of blocks, so two partial folds combine like one more fold
 * step): per row, with
 * m = max(ma, mb), l = la e^(ma-m) + lb e^(mb-m) and
 * acc = acca e^(ma-m) + accb e^(mb-m).  A side with m = -inf (no visible key)
 * contributes nothing; a row empty on both sides stays empty.
 *   a, b, out: states with equal B, Hq, Sq, D.  out may be exactly a or b
 *   (same buffers); other overlaps are not allowed. */
ra_status ra_state_merge(const ra_state* a, const ra_state* b, const ra_state* out,
                         void* stream);

/* Merge two finalized partial results of the same rows over disjoint key sets
 * ("3.6 Distributed Training II", "Vocab-parallel cross-entropy": logsumexp =
 * m + log Z, merged across shards): lse = log(e^lse_a + e^lse_b) and
 * out = out_a e^(lse_a - lse) + out_b e^(lse_b - lse), in out's dtype (round
 * to nearest even for bf16).  A side with lse = -inf contributes nothing; a
 * row empty on both sides gets out = 0, lse = -inf.
 *   out_a, out_b, out: [rows, D] of `dtype`, 16-byte aligned; lse_a, lse_b,
 *   lse: [rows] fp32.
 *   out / lse may be exactly out_a / lse_a or out_b / lse_b; other overlaps
 *   are not allowed. */
ra_status ra_merge(const void* out_a, const float* lse_a, const void* out_b, const float* lse_b,
                   void* out, float* lse, int64_t rows, int64_t D, ra_dtype dtype, void* stream);

/* ---- Vocab-parallel cross-entropy ("3.6 Distributed Training II",
 * "Vocab-parallel cross-entropy"): the loss of a row of logits z with global
 * target id t is logsumexp(z) - z[t].  With the vocab split into shards, each
 * shard reduces its columns to a row max, a sum of exponentials and the
 * target logit if it owns t; a MAX and two SUMs over the shards combine
 * them; the gradient softmax(z) - onehot(t) is split like the logits.
 * Logits are bf16 or fp32 (computed in fp32); targets are int64 ids; a target
 * outside the vocab is owned by no shard (its target logit counts as 0). */

/* One shard's statistics, in a single pass over its logits: for each row r
 * of the shard's logits [N, V_loc] (row stride ld elements, element-aligned),
 *   m[r]     = max_j z[r][j],
 *   z_sum[r] = sum_j exp(z[r][j] - m[r])   (against the shard's own max),
 *   pred[r]  = z[r][target[r] - vocab_start] if the shard owns target[r]
 *              (vocab_start <= target[r] < vocab_start + V_loc), else 0.
 * A row of -inf logits gives m = -inf, z_sum = 0.  m, z_sum, pred: [N] fp32;
 * target: [N].  N < 2^31.  No output may overlap another or an input. */
ra_status ra_vocab_ce_shard(const void* logits, int64_t ld, const int64_t* target, int64_t N,
                            int64_t V_loc, int64_t vocab_start, ra_dtype dtype, float* m,
                            float* z_sum, float* pred, void* stream);

/* Combine the statistics of t shards ([t, N] each, shard k's rows at k*N):
 * M = max_k m_k, Z = sum_k z_sum_k exp(m_k - M), P = sum_k pred_k;
 * loss[r] = M + log Z - P and, unless lse is NULL, lse[r] = M + log Z.
 * loss and lse may not overlap each other or the inputs. */
ra_status ra_vocab_ce_combine(const float* m, const float* z_sum, const float* pred, int t,
                              int64_t N, float* loss, float* lse, void* stream);

/* Gradient of scale x (the sum of the row losses) with respect to one shard's
 * logits: grad[r][j] = scale * (exp(z[r][j] - lse[r]) - [j == target[r] -
 * vocab_start]), written in `dtype` (bf16 rounded to nearest even) with row
 * stride ldg.  lse from ra_vocab_ce_combine / ra_vocab_ce; scale = 1/N gives
 * the gradient of the mean loss.  grad must not overlap the logits, target
 * or lse.
 * N x ceil(V_loc x element size / 4096) < 2^31. */
ra_status ra_vocab_ce_grad(const void* logits, int64_t ld, const int64_t* target, const float* lse,
                           int64_t N, int64_t V_loc, int64_t vocab_start, float scale,
                           ra_dtype dtype, void* grad, int64_t ldg, void* stream);

/* Bytes of workspace ra_vocab_ce needs for N rows and t shards. */
size_t ra_vocab_ce_workspace_bytes(int64_t N, int t);

/* The whole vocab-parallel cross-entropy on one GPU: logits [N, V] (dense
 * rows) split into t shards of V/t columns (V % t == 0, 1 <= t <= 1024), each
 * reduced by the shard kernel, then combined.  loss: [N] fp32; mean_loss: one
 * fp32 (device), the mean of loss summed in a fixed order (deterministic);
 * lse: [N] fp32 or NULL.  ws: at least ra_vocab_ce_workspace_bytes(N, t)
 * bytes, 256-byte aligned.  The outputs may not overlap each other, the
 * inputs or the workspace. */
ra_status ra_vocab_ce(const void* logits, const int64_t* target, int64_t N, int64_t V, int t,
                      ra_dtype dtype, float* loss, float* mean_loss, float* lse, void* ws,
                      size_t ws_bytes, void* stream);

/* ra_vocab_ce without a workspace argument, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid allocation).  It computes exactly what ra_vocab_ce computes, with
 * the same kernels, but keeps the shard statistics and partial sums in a
 * static array of the library: 8 MiB (8388608 bytes) on each GPU it runs on,
 * reserved when the library is loaded and held until the process ends; this
 * call allocates nothing.  Sizes whose scratch, ra_vocab_ce_workspace_bytes(N,
 * t), exceeds 8 MiB are rejected with RA_ERR_WORKSPACE (for t = 8 shards, N up
 * to about 87,000 rows).  Every call on one GPU shares that GPU's array, and
 * the array keeps the last call's contents: calls that overlap on one GPU (on
 * different streams, or from several threads without ordering) race, so order
 * them on one stream.  The stream must belong to the current device.  Other
 * arguments and errors as for ra_vocab_ce; RA_ERR_HIP without a current
 * device. */
ra_status ra_vocab_ce_static(const void* logits, const int64_t* target, int64_t N, int64_t V,
                             int t, ra_dtype dtype, float* loss, float* mean_loss, float* lse,
                             void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* ra_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int ra_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_H */
