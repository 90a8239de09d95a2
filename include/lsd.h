/*
 * lsd.h - C ABI of the long-sequence DiT attention library (MI355X, gfx950).
 *
 * These calls make up the hot path of one sequence-parallel DiT attention
 * layer on one GPU:
 *
 *   lsd_relayout_seq_to_head  seq-major shards -> head-major slice (Ulysses)
 *   lsd_attn_fwd              dense bidirectional attention, O and optional LSE
 *   lsd_attn_fwd_masked       the same with a key-only padding mask
 *   lsd_attn_fwd_accumulate   the same against one K/V block, merged in place
 *                             into a running (O, LSE) (Ring step)
 *   lsd_attn_merge            exact log-sum-exp merge of partial (O, LSE)
 *   lsd_cast_qkv_fp8          one FP8 cast of Q, K, V (per-head scales)
 *   lsd_attn_fwd_fp8          attention on the FP8 inputs
 *   lsd_cast_qkv_fp8_masked   the cast with a per-batch key count
 *   lsd_attn_fwd_fp8_masked   FP8 attention with a per-batch key count
 *   lsd_cast_kv_fp8           the FP8 cast of one K/V block for a Q cast earlier
 *   lsd_attn_fwd_fp8_accumulate  FP8 attention against one K/V block, merged
 *                             in place into a running (O, LSE) (Ring step)
 *   lsd_relayout_head_to_seq  head-major slices -> seq-major shard (Ulysses,
 *                             after attention)
 *
 * Conventions shared by every call
 * --------------------------------
 * - A tensor is described by an lsd_view4: a device pointer to element
 *   [0,0,0,0] plus a logical 4-d shape and strides counted in ELEMENTS.  The
 *   logical order is (B, S, H, D): batch, sequence, head, head channel.
 *   stride[3] must be 1 (head channels contiguous); the other strides are
 *   free (non-negative), so strided views such as Q, K or V inside a fused
 *   QKV projection buffer [B, S, 3, H, D] are accepted without a copy.
 * - Elements of lsd_view4 tensors are bfloat16 (16-bit) unless stated.  LSE
 *   arrays are float32, laid out [B, H, S] contiguous.
 * - Alignment: every view's data pointer and strides[0..2] must give 16-byte
 *   aligned rows (pointer % 16 == 0, stride % 8 == 0 elements, D % 8 == 0).
 * - Ownership: the caller allocates and frees all device memory.  The library
 *   allocates nothing, keeps no pointer after a call returns, and never
 *   synchronises.  Work is enqueued on `stream` (a hipStream_t; NULL is the
 *   default stream) in call order.
 * - Errors: arguments are validated on the host before any HIP call; a
 *   violation returns LSD_EINVAL (bad argument) or LSD_EUNSUPPORTED (valid
 *   request outside what the kernels implement) and nothing is enqueued.  A
 *   launch failure returns LSD_EDEVICE.  Faults inside a kernel surface at the
 *   caller's next synchronisation, as with any HIP call.  There is no
 *   fallback path: an unsupported request always fails loudly.
 *   lsd_last_error() returns a thread-local message for the last failure.
 * - Outputs may not overlap inputs (checked by address range): LSD_EINVAL.
 * - Results are deterministic: fixed reduction order.  The only atomic is
 *   the FP8 cast's per-head absolute maximum (lsd_cast_qkv_fp8), a maximum
 *   whose result does not depend on the order the updates land in.
 */
#ifndef LSD_H
#define LSD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: lsd_cast_qkv_fp8 stores Q's scale amax (a power-of-two logit factor)
 *    in place of Q's plain amax; signatures unchanged from 1.
 * 3: adds lsd_cast_qkv_fp8_masked and lsd_attn_fwd_fp8_masked (the key-length
 *    mask on the FP8 path), lsd_attn_fwd_fp8_accumulate (the fused Ring step
 *    on FP8 inputs) and lsd_cast_kv_fp8 (the cast of one K/V block against a
 *    given Q scale); earlier entry points unchanged. */
#define LSD_ABI_VERSION 3

typedef enum lsd_status {
  LSD_OK = 0,
  LSD_EINVAL = 1,
  LSD_EUNSUPPORTED = 2,
  LSD_EDEVICE = 3
} lsd_status;

typedef struct lsd_view4 {
  void* data;        /* device pointer to element [0,0,0,0] */
  int64_t shape[4];  /* (B, S, H, D) */
  int64_t stride[4]; /* element strides; stride[3] == 1 unless stated */
} lsd_view4;

/* LSD_ABI_VERSION of the built library. */
int lsd_abi_version(void);

/* Message for the last failed call on this thread ("" if none). */
const char* lsd_last_error(void);

/*
 * Dense, unmasked, bidirectional multi-head attention with log-sum-exp.
 *
 * Defined by "Scaling Video Generation Across NVL72 rack with TensorRT-LLM":
 * "The Scaling Challenge in Video Generation" (every denoising step attends
 * over the whole sequence, no causal mask) and "Context Parallelism >
 * Attention2D Parallelism > Local Attention" (the inner backend returns the
 * partial output [B, S_q, H, D] and the LSE [B, H, S_q] of its pass).
 *
 *   q   (B, S_q,  H, D) bf16        k, v (B, S_kv, H, D) bf16
 *   o   (B, S_q,  H, D) bf16, written
 *   lse float32 [B, H, S_q] contiguous, written if non-NULL
 *
 * For each (b, h, i):  s_ij = scale * q_i . k_j,
 *   LSE_i = ln sum_j exp(s_ij)   (natural log of the scaled logits),
 *   O_i   = sum_j exp(s_ij - LSE_i) v_j, rounded to bf16 (nearest-even).
 * S_q and S_kv may differ (a query block against a key/value block).
 * S_kv == 0 gives O = 0 and LSE = -inf.  Zero-sized B, S_q or H is a no-op.
 * softmax_scale <= 0 (or NaN) selects 1/sqrt(D); +inf is rejected.
 *
 * v may be given in either layout, told apart by its strides:
 *   natural          stride[3] == 1 (each token's channels contiguous);
 *   token-contiguous stride[1] == 1 and stride[3] = row pitch: each
 *                    channel's S_kv keys form one row (storage [B, H, D, pitch]
 *                    in the usual case).  The pitch must be at least S_kv, a
 *                    multiple of 8 and below 2^23; stride[0] and stride[2]
 *                    multiples of 8.  Only keys below S_kv (below kv_lens[b]
 *                    in the masked calls) are read, so row padding may hold
 *                    anything.  This is the layout the kernel stages straight
 *                    into LDS, the faster of the two; results are identical.
 * All other strides (and every stride but the unit one of v) must be multiples
 * of 8 elements and the data pointers 16-byte aligned (LSD_EINVAL otherwise).
 * D must be 64 or 128, and the sequence stride of k (and of a natural v) must
 * be below 2^24 elements (LSD_EUNSUPPORTED otherwise).  The device must be
 * gfx950 (LSD_EUNSUPPORTED otherwise).
 */
lsd_status lsd_attn_fwd(const lsd_view4* q, const lsd_view4* k, const lsd_view4* v,
                        const lsd_view4* o, float* lse, float softmax_scale, void* stream);

/*
 * lsd_attn_fwd with a key-only padding mask: batch entry b attends only its
 * first kv_lens[b] keys; the keys after them (padding) get weight exactly 0,
 * are never read, and may hold anything (NaN included).  Every query row,
 * padded rows included, attends all valid keys of its batch entry, so no row
 * is NaN.  A batch entry with kv_lens[b] == 0 gives O = 0 and LSE = -inf.
 *
 * Defined by "How 8 GPUs split tokens: what LTX-2's sequence-parallel all2all
 * moves", "Data flow": the sequence is padded to a multiple of the parallel
 * degree and a key-only mask (valid keys 1, padding 0, broadcast over batch
 * and queries) keeps the padding out of attention; padded query rows see all
 * valid keys.  Per-batch lengths generalise the single mask to a batch of
 * sequences of different lengths.
 *
 *   kv_lens  int32 device array of B entries, 4-byte aligned; values are
 *            clamped to [0, S_kv] in the kernel (the host cannot read them).
 *
 * Everything else as for lsd_attn_fwd.
 */
lsd_status lsd_attn_fwd_masked(const lsd_view4* q, const lsd_view4* k, const lsd_view4* v, const int32_t* kv_lens,
                               const lsd_view4* o, float* lse, float softmax_scale, void* stream);

/*
 * One Ring step with the merge folded in: attention of q against one key/value
 * block, merged into a running result in place.
 *
 * Defined by "Scaling Video Generation Across NVL72 rack with TensorRT-LLM",
 * "Context Parallelism > Ring Attention" (each arriving K/V block's partial
 * result is merged into the running output with the fp32 online-softmax
 * recurrence, so no separate combine pass is needed) and "Limitations and
 * Future Work" (folding the combine into the attention kernel).
 *
 *   q, k, v  as for lsd_attn_fwd (k, v: this step's key/value block)
 *   kv_lens  NULL, or the key-only padding mask of lsd_attn_fwd_masked for
 *            this block (batch entry b uses the block's first kv_lens[b] keys)
 *   o_acc    float32 [B, S_q, H, D] contiguous, 16-byte aligned: read, written
 *   lse_acc  float32 [B, H, S_q] contiguous: read, written
 *   o        (B, S_q, H, D) bf16, written if non-NULL: the updated running
 *            output rounded to bf16 (pass it on the last step)
 *
 * With (O_b, LSE_b) this block's attention result (as lsd_attn_fwd computes
 * it, kept in float32), M = max(LSE_acc, LSE_b) and w = exp(LSE - M):
 *   O_acc   <- (w_acc O_acc + w_b O_b) / (w_acc + w_b)
 *   LSE_acc <- M + ln(w_acc + w_b)
 * Start a sequence of steps with lse_acc = -inf: where LSE_acc = -inf the
 * running O_acc is not read (it may hold anything).  A block with no keys
 * (S_kv == 0) leaves o_acc and lse_acc unchanged (and writes their bf16 form,
 * 0 where LSE_acc = -inf, to o).  lse_acc must hold LSEs or -inf (no NaN).
 * Other rules as for lsd_attn_fwd; o_acc, lse_acc and o may not overlap each
 * other or an input.
 */
lsd_status lsd_attn_fwd_accumulate(const lsd_view4* q, const lsd_view4* k, const lsd_view4* v,
                                   const int32_t* kv_lens, float* o_acc, float* lse_acc, const lsd_view4* o,
                                   float softmax_scale, void* stream);

/*
 * Exact merge of n partial attention results over disjoint key spans.
 *
 * Defined by "Scaling Video Generation Across NVL72 rack with TensorRT-LLM",
 * "Context Parallelism > Ring Attention" (online-softmax merge of per-block
 * outputs and LSE) and "Attention2D Parallelism > Merge phase" (one batched
 * combine of the received (output, LSE) pairs).
 *
 *   o_parts[i]   (B, S, H, D) bf16, i = 0..n-1 (any strides as above)
 *   lse_parts[i] float32 [B, H, S] contiguous
 *   o_out        (B, S, H, D) bf16, written
 *   lse_out      float32 [B, H, S] contiguous, written if non-NULL
 *
 * With M = max_i LSE_i and w_i = exp(LSE_i - M):
 *   LSE = M + ln sum_i w_i,   O = (sum_i w_i O_i) / sum_i w_i  (float32 math,
 *   partials summed in order i = 0..n-1, O rounded to bf16 nearest-even).
 * Where every LSE_i is -inf: O = 0, LSE = -inf.  1 <= n <= 16.
 * o_out and lse_out may not overlap any input.
 */
lsd_status lsd_attn_merge(int n, const lsd_view4* o_parts, const float* const* lse_parts,
                          const lsd_view4* o_out, float* lse_out, void* stream);

/*
 * One FP8 cast pass over Q, K and V, producing the inputs of lsd_attn_fwd_fp8.
 *
 * Defined by "Scaling Video Generation Across NVL72 rack with TensorRT-LLM",
 * "Ulysses Parallelism > Fused vs. unfused QKV all-to-all": the stacked QKV
 * buffer gets a single FP8 cast pass before the attention kernel (not three
 * casts), landing in a layout the kernel reads without another copy.
 *
 *   src   3 bf16 views (B, S, H, D): Q, K, V (e.g. strided views of a fused
 *         [B, S, 3, H, D] buffer), one shape, D = 128
 *   dst   3 FP8 E4M3 views (B, S, H, D), one byte per element, strides in
 *         bytes: dst[0] (Q) and dst[1] (K) with channels contiguous
 *         (stride[3] = 1); dst[2] (V) stored transposed, tokens contiguous
 *         (stride[1] = 1), stride[3] = row pitch of one (b, h, d) row, at
 *         least S rounded up to 64: the cast also writes zero codes for the
 *         tokens S .. that bound (each row must be allocated that far)
 *   amax  float32 [3, B, H]: per (tensor, batch, head) the scale amax the
 *         codes use, written: for K and V max |x| over tokens and channels;
 *         for Q the smallest value amax_q' >= max |q| for which
 *         log2(e)/sqrt(128) * (amax_q'/448) * (amax_k/448) is a power of two
 *         (float32 steps: base = log2(e)/sqrt(128) * (amax_k/448),
 *         t = base * (amax_q/448), 2^e the smallest power of two >= t,
 *         amax_q' = (2^e / base) * 448, from 2^(e+1) if that falls below
 *         amax_q; it lies in [amax_q, 2 amax_q)); a zero amax_q or amax_k,
 *         or a result that is not finite, keeps amax_q
 *
 * code = E4M3(x * (448 / amax)): the product rounded to float32, the code to
 * nearest, ties to even (OCP E4M3: largest finite 448); a head whose amax is
 * 0 uses factor 1.  The dequantised value is code * (amax / 448).  The Q scale
 * makes lsd_attn_fwd_fp8's logit factor at the default softmax scale an exact
 * power of two, which that kernel applies on the matrix cores.  All other
 * byte strides and pointers must be multiples of 16.  Deterministic (the amax
 * reduction takes maxima, which do not depend on order).  Four launches on
 * `stream`.
 */
lsd_status lsd_cast_qkv_fp8(const lsd_view4* src, const lsd_view4* dst, float* amax, void* stream);

/*
 * Dense bidirectional attention over FP8 inputs: the attention of the
 * dequantised values, computed on FP8 matrix cores.
 *
 * Defined as lsd_attn_fwd of q = code_q * s_q, k = code_k * s_k,
 * v = code_v * s_v with s = amax / 448 per (b, h) ("Scaling Video Generation
 * Across NVL72 rack with TensorRT-LLM", "Ulysses Parallelism > Fused vs.
 * unfused QKV all-to-all" and "The Scaling Challenge in Video Generation").
 *
 *   q8, k8   E4M3 (B, S_q, H, D) and (B, S_kv, H, D) views, channels
 *            contiguous, as lsd_cast_qkv_fp8 writes them
 *   v8       E4M3 (B, S_kv, H, D) view stored transposed (tokens contiguous,
 *            stride[3] = row pitch); every row must be readable, with finite
 *            codes, up to S_kv rounded up to 64 tokens from the view's start
 *            (the cast's padded rows satisfy this for views that start at a
 *            multiple of 64 tokens), and stride[3] must be at least that
 *   q_amax, k_amax, v_amax  float32 [B, H]: the scale amax of each tensor
 *            (as lsd_cast_qkv_fp8 writes them; any positive values work)
 *   o        bf16 (B, S_q, H, D), written;  lse  float32 [B, H, S_q] or NULL
 *
 * D = 128 only.  The softmax weights are rounded to E4M3 for the PV product
 * (the row sums stay float32), so O carries an error of up to 2^-4 of
 * sum_j p_j |v_j| / l (see the design notes for the full bound); LSE is as
 * exact as in lsd_attn_fwd.  When scale * log2(e) * (q_amax/448) *
 * (k_amax/448) is within 2^-20 of a power of two, that power of two is used
 * as the logit factor (a relative change of at most 2^-20).  S_kv == 0 gives
 * O = 0, LSE = -inf.
 */
lsd_status lsd_attn_fwd_fp8(const lsd_view4* q8, const lsd_view4* k8, const lsd_view4* v8, const float* q_amax,
                            const float* k_amax, const float* v_amax, const lsd_view4* o, float* lse,
                            float softmax_scale, void* stream);

/*
 * The FP8 cast and FP8 attention with the key-only padding mask of
 * lsd_attn_fwd_masked (defined by "How 8 GPUs split tokens: what LTX-2's
 * sequence-parallel all2all moves", "Data flow": padding keys get zero
 * weight, every query row sees all valid keys of its batch entry), combined
 * with the single FP8 cast of "Scaling Video Generation Across NVL72 rack
 * with TensorRT-LLM", "Ulysses Parallelism > Fused vs. unfused QKV
 * all-to-all"; the per-head scales then come from the valid tokens alone.
 *
 *   kv_lens  int32 device array of B entries, 4-byte aligned, not NULL;
 *            batch entry b has kv_lens[b] valid keys (clamped to [0, S]);
 *            it may not overlap any output
 *
 * lsd_cast_qkv_fp8_masked: as lsd_cast_qkv_fp8, except that K's and V's amax
 * are taken over the valid tokens only (0 for an entry without keys, which
 * also leaves Q's amax unadjusted), V's codes of the tokens from kv_lens[b]
 * to the padded row end are zero, and K's codes of the tokens from
 * kv_lens[b] on are not written.  Padding may hold any bits (NaN included).
 *
 * lsd_attn_fwd_fp8_masked: as lsd_attn_fwd_fp8 over the first kv_lens[b] keys
 * of batch entry b; K rows past them are not read, V rows are read up to
 * kv_lens[b] rounded up to 64 tokens and must hold finite codes there (the
 * masked cast writes zeros).  An entry with kv_lens[b] == 0 gives O = 0 and
 * LSE = -inf.
 */
lsd_status lsd_cast_qkv_fp8_masked(const lsd_view4* src, const lsd_view4* dst, float* amax, const int32_t* kv_lens,
                                   void* stream);
lsd_status lsd_attn_fwd_fp8_masked(const lsd_view4* q8, const lsd_view4* k8, const lsd_view4* v8,
                                   const float* q_amax, const float* k_amax, const float* v_amax,
                                   const int32_t* kv_lens, const lsd_view4* o, float* lse, float softmax_scale,
                                   void* stream);

/*
 * One Ring step on FP8 inputs with the merge folded in: lsd_attn_fwd_fp8 of q8
 * against one key/value block (its codes and scales as the FP8 cast of that
 * block writes them), merged into a running result in place, exactly as
 * lsd_attn_fwd_accumulate merges (same rules for o_acc, lse_acc, o, kv_lens
 * and an empty block).  Defined by "Scaling Video Generation Across NVL72 rack
 * with TensorRT-LLM", "Context Parallelism > Ring Attention" (each arriving
 * block's partial result merged into the running output with the fp32
 * online-softmax recurrence) and "Limitations and Future Work" (the combine
 * folded into the attention kernel), on the FP8 inputs of "Ulysses
 * Parallelism > Fused vs. unfused QKV all-to-all".
 *
 *   q8, k8, v8, q_amax, k_amax, v_amax  as for lsd_attn_fwd_fp8 (k8, v8 and
 *            their scales: this step's block)
 *   kv_lens  NULL, or this block's valid keys per batch entry (as for
 *            lsd_attn_fwd_fp8_masked)
 *   o_acc    float32 [B, S_q, H, D] contiguous, 16-byte aligned: read, written
 *   lse_acc  float32 [B, H, S_q] contiguous: read, written
 *   o        (B, S_q, H, D) bf16, written if non-NULL (the updated running
 *            output in bf16)
 *
 * The block's own result carries the FP8 error of lsd_attn_fwd_fp8; the merge
 * is the float32 arithmetic of lsd_attn_fwd_accumulate.
 */
/*
 * The FP8 cast of one key/value block for a query cast earlier (a Ring step's
 * block): as lsd_cast_qkv_fp8 (or lsd_cast_qkv_fp8_masked with kv_lens) for K
 * and V, except that Q is not cast and K's scale amax, not Q's, is adjusted:
 * the smallest value amax_k' >= max |k| for which
 * log2(e)/sqrt(128) * (q_scale_amax/448) * (amax_k'/448) is a power of two
 * (the rule of lsd_cast_qkv_fp8 for Q with the two roles swapped; the factor
 * is symmetric in them).  With it, lsd_attn_fwd_fp8 at the default softmax
 * scale applies the logit factor exactly on the matrix cores for every block,
 * although each block has its own scales.
 *
 *   src           2 bf16 views (B, S, H, D): K, V of the block, one shape
 *   dst           2 FP8 views as dst[1] and dst[2] of lsd_cast_qkv_fp8
 *   amax          float32 [3, B, H], written: [0] zero (no Q), [1] K's scale
 *                 amax, [2] V's amax
 *   q_scale_amax  float32 [B, H], not NULL: the query's scale amax (amax[0]
 *                 of the query's lsd_cast_qkv_fp8)
 *   kv_lens       NULL, or the block's valid keys per batch entry (as for
 *                 lsd_cast_qkv_fp8_masked)
 */
lsd_status lsd_cast_kv_fp8(const lsd_view4* src, const lsd_view4* dst, float* amax, const float* q_scale_amax,
                           const int32_t* kv_lens, void* stream);

lsd_status lsd_attn_fwd_fp8_accumulate(const lsd_view4* q8, const lsd_view4* k8, const lsd_view4* v8,
                                       const float* q_amax, const float* k_amax, const float* v_amax,
                                       const int32_t* kv_lens, float* o_acc, float* lse_acc, const lsd_view4* o,
                                       float softmax_scale, void* stream);

/*
 * Ulysses sequence-major -> head-major relayout for one destination rank.
 *
 * Defined by "Scaling Video Generation Across NVL72 rack with TensorRT-LLM",
 * "Ulysses Parallelism" ([B, S/P, H, D] -> [B, S, H/P, D]; P must divide H;
 * the fused variant moves Q, K and V together), and by "CUDA IPC Ulysses"
 * (TeleFuser), sections "Baseline and bottleneck" and "Strided Copy Engine
 * scatter" (the fused projection's V is read as a strided view, each token's
 * heads and channels contiguous, written straight into the final
 * (B, S_global, H_local, D) layout).
 *
 *   src  n_tensors * P views, index t*P + p: sequence shard p of tensor t,
 *        each (B, S_loc, H, D); all of one shape.
 *   dst  n_tensors views, each (B, P*S_loc, H/P, D), written.
 *
 *   dst[t][b, p*S_loc + s, j, :] = src[t*P + p][b, s, rank*(H/P) + j, :]
 *
 * A destination may instead be token-contiguous (stride[1] == 1, stride[3] =
 * row pitch, as lsd_attn_fwd accepts V): each channel's P*S_loc tokens are
 * then written as one row, which lets attention stage V straight into LDS.
 * Its pitch must be at least P*S_loc, a multiple of 8 and below 2^23, rows and
 * heads may not overlap (stride[2] >= D*stride[3], stride[0] >= (H/P)*stride[2])
 * and D must be a multiple of 64; row padding is never written.
 * A pure 16-bit copy: every bit pattern (NaN payloads, -0) is preserved.
 * 1 <= n_tensors <= 3, 1 <= P <= 16, 0 <= rank < P, H % P == 0 (LSD_EINVAL
 * otherwise).  Destinations may not overlap any source or each other.
 */
lsd_status lsd_relayout_seq_to_head(int n_tensors, int P, int rank, const lsd_view4* src,
                                    const lsd_view4* dst, void* stream);

/*
 * Ulysses head-major -> sequence-major relayout for one destination rank: the
 * inverse of lsd_relayout_seq_to_head, run on the attention output.
 *
 * Defined by "Scaling Video Generation Across NVL72 rack with TensorRT-LLM",
 * "Ulysses Parallelism" and its Figure 2 (after the full-sequence attention
 * the [B, S, H/P, D] head slices are converted back to the [B, S/P, H, D]
 * sequence shards the MLP works on), and by "How 8 GPUs split tokens: what
 * LTX-2's sequence-parallel all2all moves", "Precise statement" (the round
 * trip through both exchanges returns every byte).
 *
 *   src  n_tensors * P views, index t*P + r: rank r's head slice of tensor t,
 *        each (B, P*S_loc, H_loc, D); all of one shape.
 *   dst  n_tensors views, each (B, S_loc, P*H_loc, D), written.
 *
 *   dst[t][b, s, r*H_loc + j, :] = src[t*P + r][b, rank*S_loc + s, j, :]
 *
 * So lsd_relayout_head_to_seq(rank p) applied to the P outputs of
 * lsd_relayout_seq_to_head(rank 0..P-1) returns sequence shard p bit for bit.
 * A pure 16-bit copy.  1 <= n_tensors <= 3, 1 <= P <= 16, 0 <= rank < P, and
 * P must divide the slices' sequence length (LSD_EINVAL otherwise).
 * Destinations may not overlap any source or each other.
 */
lsd_status lsd_relayout_head_to_seq(int n_tensors, int P, int rank, const lsd_view4* src,
                                    const lsd_view4* dst, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LSD_H */
