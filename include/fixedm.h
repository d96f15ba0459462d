/*
 * fixedm.h - C ABI of the fixed-m ("const-max") attention forward library (gfx950).
 *
 * Sources, cited by page title and section:
 *   [CM] "Kernel reference: ring_attention_const_max_fwd const-max ring attention"
 *        (AWS Neuron documentation page)
 *   [FM] "feat(attention): fixed-m splash attention kernel with dynamic bounds and
 *        safety fallbacks" (maxdiffusion pull request #477)
 *   [UR] "feat(attention): 2D Ulysses+Ring attention with Global Virtual K-Centering"
 *        (maxdiffusion pull request #478)
 *
 * What the library computes: non-causal softmax attention O = softmax(s Q K^T) V where,
 * for every (batch, head, q-block) that passes the gate, the online-softmax running max
 * is replaced by a fixed integer shift m = ceil(U) - C(N) and the numerator and the
 * row sum accumulate in fp32 by pure addition across K/V chunks ([FM] Summary; [CM]
 * "A static bound makes the ring reduction pure addition").  Blocks that fail the gate
 * take an exact online-softmax body instead ([UR] Summary, "Cross-Ring Safety Fallback").
 * One final O = acc / l normalises ([CM] "Accumulate, then normalize once").
 *
 * Call sequence (one rank of the ring, on one GPU):
 *   fixedm_bounds      once per forward: norms, k_mean, U, m, eligibility;
 *   fixedm_run_init    once per forward: resets the host-side ring state;
 *   fixedm_attn_fwd    once per visiting K/V chunk (or once with several chunks);
 *   fixedm_finalize    once (or more): O = acc / l, optional log-sum-exp;
 * or, for the last chunks of the run, fixedm_attn_fwd_final in place of the last
 * fixedm_attn_fwd and fixedm_finalize (the final fold and the normalisation in one pass).
 *
 * Conventions shared by every entry point:
 *   - Tensors are described by fixedm_tensor: a device pointer plus element strides for
 *     the batch, sequence and head axes; the head_dim axis is contiguous (stride 1).
 *     Layout is token-major [B, S, H, D] as in the [CM] Interface table, but any
 *     non-negative strides are accepted, within these limits: ptr must be 16-byte aligned,
 *     every stride a multiple of 8 elements (bf16) or 4 elements (fp32), and a bf16
 *     tensor's sequence stride at most 2^26 elements (FIXEDM_ERR_UNSUPPORTED_SHAPE
 *     otherwise).
 *   - Every device pointer and the stream belong to the caller.  The library never
 *     allocates, frees or synchronises, and keeps no pointer after a call returns.  The
 *     scratch buffers it writes (bounds buffer, workspace) come with their byte sizes,
 *     checked against the problem before anything is enqueued.
 *     Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = default stream).
 *   - Host-checkable errors are returned before anything is enqueued.  A failed launch
 *     returns FIXEDM_ERR_HIP.  Data-dependent ineligibility is never an error: it selects
 *     the exact fallback body ([FM] commit message: contracts fail loudly, data picks the
 *     path; [CM] Best practices: no selector for the only correct path).
 *   - Only bf16 and fp32 inputs exist in this ABI.  fp16/fp8 would overflow the fixed-m
 *     exponent window ([FM] commit message, dtype safety) and have no enum value.
 */
#ifndef FIXEDM_H
#define FIXEDM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FIXEDM_ABI_VERSION 2

typedef enum {
  FIXEDM_OK = 0,
  FIXEDM_ERR_INVALID_ARGUMENT = -1,  /* null pointer, negative size, bad enum, bad abi_version */
  FIXEDM_ERR_UNSUPPORTED_DTYPE = -2, /* dtype not bf16/fp32, or a path that lacks it */
  FIXEDM_ERR_UNSUPPORTED_SHAPE = -3, /* head_dim, q_block, alignment or strides not supported */
  FIXEDM_ERR_BOUNDS_MISMATCH = -4,   /* descriptor token/dims disagree with the call */
  FIXEDM_ERR_STATE = -5,             /* ring state misuse, e.g. finalize before all N keys */
  FIXEDM_ERR_HIP = -6                /* a HIP launch or runtime call failed */
} fixedm_status;

typedef enum { FIXEDM_BF16 = 1, FIXEDM_F32 = 2 } fixedm_dtype;

/* Virtual K-centring ([FM] Summary; [UR] Summary).  The centring mode is recorded in the
 * bounds descriptor and used by both the bound and the logits, so the unsound pairing of
 * a raw-key bound with centred logits ([FM] "This PR is additive") cannot be expressed. */
typedef enum {
  FIXEDM_CENTER_NONE = 0,     /* k_mean = 0 */
  FIXEDM_CENTER_SUPPLIED = 1, /* caller's fp32 [B, H, D] mean */
  FIXEDM_CENTER_COMPUTE = 2   /* mean of the real keys of all chunks, fp64 sum, fp32 result */
} fixedm_center;

/* Granularity of the fixed shift m.  BLOCK: one m per (batch, head, q-block) ([FM]
 * Summary).  ROW: one m per query row from that row's own norm, the per-query-row bound of
 * [CM] "Picking a max that is safe without measuring it" (Best practices: "Give each query
 * row its own bound"), in the same base-2 integer form m_i = ceil(U_i) - C(N).  In both
 * modes eligibility is decided per q-block: the body is chosen per block, and a block
 * passes when its loudest row does. */
typedef enum { FIXEDM_SHIFT_BLOCK = 0, FIXEDM_SHIFT_ROW = 1 } fixedm_shift;

typedef struct {
  const void* ptr;  /* device pointer to element [0, 0, 0, 0] */
  int64_t stride_b; /* element strides; the head_dim axis has stride 1 */
  int64_t stride_s;
  int64_t stride_h;
} fixedm_tensor;

typedef struct {
  int32_t abi_version;   /* must be FIXEDM_ABI_VERSION */
  int32_t dtype;         /* fixedm_dtype of q, k and v */
  int64_t batch;         /* B >= 1; B x H <= 65,535 */
  int64_t heads;         /* H >= 1; MHA only (K/V have the same H as Q) */
  int64_t head_dim;      /* D: 128 (bf16 and fp32) or 64 (fp32 only) */
  int64_t sq;            /* resident query rows, 1 .. 2^30; B x H x ceil(sq / 256) < 2^31 */
  int64_t sk_total;      /* N: real keys over all chunks, 1 .. 2^38 (bf16: 2^35), unpadded ([UR] Summary) */
  int64_t q_block;       /* rows per shift/eligibility block: positive multiple of 64 */
  float softmax_scale;   /* s; 0 selects fp32(1/sqrt(D)) ([CM] Interface table) */
  int32_t center;        /* fixedm_center */
  int32_t shift;         /* fixedm_shift */
} fixedm_problem;

/* Filled by fixedm_bounds; the caller owns it and must not modify it afterwards. */
typedef struct {
  fixedm_problem p;      /* copy of the problem, softmax_scale resolved */
  int32_t log2_n;        /* ceil(log2 N) */
  int32_t C;             /* C(N) = 127 - ceil(log2 N) - ceil(log2 256) ([FM] Summary) */
  int32_t W;             /* W(N) = C(N) + 125 */
  int32_t gate;          /* floor(W / 2) ([FM] "Why the gate is halved") */
  int64_t n_qblocks;     /* ceil(sq / q_block) */
  float alpha;           /* fp32(softmax_scale * log2(e)): base-2 logit factor */
  int32_t reserved;
  void* dev;             /* caller's device buffer of fixedm_bounds_bytes() bytes */
  uint64_t token;        /* binds run states and calls to this descriptor */
} fixedm_bounds_t;

/* Host-side ring state: the first chunk visit initialises the accumulator, later
 * visits add to it ([CM] Overview ring figure; "Accumulate, then normalize once"). */
typedef struct {
  uint64_t token;
  int64_t kv_visited;    /* keys folded in so far */
  int32_t calls;         /* fixedm_attn_fwd / fixedm_attn_fwd_final calls so far */
  int32_t finalized;     /* 1 after fixedm_attn_fwd_final: the run is complete and the
                            workspace no longer holds its whole result */
} fixedm_run_t;

/* Byte offsets of the arrays fixedm_bounds writes into the descriptor's device buffer.
 * m: int32 [B, H, nQB]; elig: uint8 [B, H, nQB] (1 = fixed-m body); u: fp64 [B, H, nQB];
 * q2: fp64 [B, H, nQB] (max of sum_d q^2 over the block's real rows); k2: fp64 [B, H]
 * (max of sum_d (k - k_mean)^2 over all keys); k_mean: fp32 [B, H, D]; v_bad: int32
 * (0 when every V element has |v| <= 256, else the fp32 bit pattern of the largest |v|,
 * inf and NaN included; v_ok = (v_bad == 0)).  With
 * shift == FIXEDM_SHIFT_ROW also m_row: int32 [B, H, sq] (m_i = ceil(u_i) - C), q2_row:
 * fp64 [B, H, sq] (sum_d q_id^2) and u_row: fp64 [B, H, sq] (alpha64 * sqrt(q2_i * k2));
 * in BLOCK mode these three arrays are empty (their offsets equal the next one's). */
typedef struct {
  size_t m, elig, u, q2, k2, k_mean, v_bad, m_row, q2_row, u_row, scratch, total;
} fixedm_bounds_layout_t;

/* Size of the device buffer fixedm_bounds needs, or 0 if the problem is invalid. */
size_t fixedm_bounds_bytes(const fixedm_problem* p);

/* Offsets of the arrays inside that buffer.  Returns FIXEDM_ERR_* on an invalid problem. */
fixedm_status fixedm_bounds_layout(const fixedm_problem* p, fixedm_bounds_layout_t* out);

/* Size of the accumulator workspace fixedm_attn_fwd/fixedm_finalize use (fp32 acc, row
 * sum l and row shift r for every padded query row; for bf16 problems also the same three
 * for the key-range parts of up to 255 split tail tiles), or 0 if the problem is invalid.
 * How the bf16 kernel splits its last partial round of tiles depends on the problem and on
 * the device's compute-unit count, so a run's fixedm_attn_fwd and fixedm_finalize calls
 * must use the same device (they always do for one workspace in practice). */
size_t fixedm_workspace_bytes(const fixedm_problem* p);

/* Host-only constants of [FM] Summary for n >= 1 keys:
 * log2_n = ceil(log2 n), C = 127 - log2_n - 8, W = C + 125, gate = floor(W / 2).
 * Any output pointer may be NULL.  n < 1 -> FIXEDM_ERR_INVALID_ARGUMENT. */
fixedm_status fixedm_constants(int64_t n, int32_t* log2_n, int32_t* C, int32_t* W,
                               int32_t* gate);

/* Bounds and gate ([FM] Summary; [CM] "Picking a max that is safe without measuring it",
 * "Transpose prologue with fused norms"; [UR] Summary, merged norm reduction):
 *   k_mean  per centring mode (COMPUTE: fp32(fp64 sum of all real keys / N));
 *   q2[b,h,beta] = max over the block's real rows of sum_d q_d^2        (fp64);
 *   k2[b,h]      = max over all keys of all chunks of sum_d (k_d - k_mean_d)^2 (fp64);
 *   u  = alpha64 * sqrt(q2 * k2), alpha64 = fp64(s) * log2(e);  m = ceil(u) - C;
 *   elig = (no |v| > 256 anywhere in V) && u <= gate && u finite;
 *   shift == ROW: per query row also u_i = alpha64 * sqrt(q2_i * k2), m_i = ceil(u_i) - C,
 *   and the attention calls shift row i by m_i (eligibility stays the block's).
 * q: [B, sq, H, D]; k_chunks/v_chunks: n_chunks tensors of [B, chunk_len[c], H, D];
 * sum(chunk_len) must equal p->sk_total.  k_mean_in: device fp32 [B, H, D] contiguous,
 * required iff center == SUPPLIED.  bounds_dev: device buffer of bounds_dev_bytes >=
 * fixedm_bounds_bytes(p) bytes, 256-byte aligned (a smaller size ->
 * FIXEDM_ERR_INVALID_ARGUMENT).  On success *out describes the result (valid once the stream
 * reaches this point).  Enqueues 4-6 kernels; no host synchronisation. */
fixedm_status fixedm_bounds(const fixedm_problem* p, fixedm_tensor q,
                            const fixedm_tensor* k_chunks, const fixedm_tensor* v_chunks,
                            const int64_t* chunk_len, int32_t n_chunks,
                            const float* k_mean_in, void* bounds_dev,
                            size_t bounds_dev_bytes, fixedm_bounds_t* out, void* stream);

/* fixedm_bounds for callers that cannot allocate memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same computation and results, with
 * the scratch fixedm_bounds keeps at the end of its buffer (the key-mean partial sums of
 * COMPUTE centring) held instead in one static device array of 24 MiB per GPU, allocated
 * when the library's code is loaded on that GPU and kept until the process ends.  bounds_dev
 * needs only the output arrays: bounds_dev_bytes >= the `scratch` offset of
 * fixedm_bounds_layout.  Problems whose partial sums cannot fit that array even with a
 * single key slab (batch x heads x head_dim x 12 bytes above 24 MiB) are rejected with
 * FIXEDM_ERR_UNSUPPORTED_SHAPE.  Allocates nothing and calls no allocating routine; a failed
 * lookup of the array's address returns FIXEDM_ERR_HIP.  Every call on one GPU uses the same
 * array: calls that overlap on one GPU (other streams, other host threads) race; calls on
 * one stream, or separated by synchronisation, are safe.  The descriptor it fills is used
 * exactly like fixedm_bounds's. */
fixedm_status fixedm_bounds_static(const fixedm_problem* p, fixedm_tensor q,
                                   const fixedm_tensor* k_chunks, const fixedm_tensor* v_chunks,
                                   const int64_t* chunk_len, int32_t n_chunks,
                                   const float* k_mean_in, void* bounds_dev,
                                   size_t bounds_dev_bytes, fixedm_bounds_t* out, void* stream);

/* Starts a new ring pass over the descriptor's K/V: zero keys visited. */
fixedm_status fixedm_run_init(const fixedm_bounds_t* bounds, fixedm_run_t* run);

/* One or more ring steps ([CM] Overview ring figure, "The ring loop"): folds n_chunks
 * K/V chunks (in the given order) into the caller's workspace.  Up to 8 chunks of one call
 * are folded by one launch with the accumulators resident in registers across them.  The first keys of a run
 * initialise the workspace, later ones add to it: pure addition for eligible blocks,
 * the online-softmax rescale merge for the others.  q: [B, sq, H, D] (the same rows the
 * bounds were computed from); chunks as in fixedm_bounds.  workspace: device buffer of
 * workspace_bytes >= fixedm_workspace_bytes() bytes, 256-byte aligned (a smaller size ->
 * FIXEDM_ERR_INVALID_ARGUMENT).  Errors: FIXEDM_ERR_BOUNDS_MISMATCH
 * if run->token does not match the descriptor, FIXEDM_ERR_STATE if the keys visited
 * would exceed sk_total or the run was completed by fixedm_attn_fwd_final.  Updates *run
 * on success. */
fixedm_status fixedm_attn_fwd(const fixedm_bounds_t* bounds, fixedm_run_t* run,
                              fixedm_tensor q, const fixedm_tensor* k_chunks,
                              const fixedm_tensor* v_chunks, const int64_t* chunk_len,
                              int32_t n_chunks, void* workspace, size_t workspace_bytes,
                              void* stream);

/* The last ring step(s) of a run fused with the finalize ([CM] "Accumulate, then normalize
 * once": the last step folds and normalises in one pass; "The ring loop").  Folds
 * n_chunks K/V chunks like fixedm_attn_fwd, which must bring the run to sk_total keys
 * (FIXEDM_ERR_STATE otherwise; n_chunks may be 0 with all keys already visited), and
 * writes out and lse exactly as fixedm_finalize describes.  On the bf16 path the chunks of
 * the call are folded with the accumulators resident in registers, and each query tile
 * writes its output rows straight from them; only the split tail tiles (the key-range
 * parts of the last partial round of tiles) pass through the workspace and a finalize
 * over those tiles.  On the fp32 path it is fixedm_attn_fwd followed by fixedm_finalize.
 * Arguments as in those two calls.  Sets run->finalized: a later fixedm_finalize or
 * fixedm_attn_fwd on this run returns FIXEDM_ERR_STATE. */
fixedm_status fixedm_attn_fwd_final(const fixedm_bounds_t* bounds, fixedm_run_t* run,
                                    fixedm_tensor q, const fixedm_tensor* k_chunks,
                                    const fixedm_tensor* v_chunks, const int64_t* chunk_len,
                                    int32_t n_chunks, void* workspace, size_t workspace_bytes,
                                    fixedm_tensor out,
                                    int32_t out_dtype, float* lse, void* stream);

/* O = acc / l (in fp32 as acc times the correctly rounded 1 / l, within 1.5 ulp of the
 * quotient; fixedm_attn_fwd_final forms it the same way), cast to out_dtype (bf16 by
 * round-to-nearest-even, a NaN staying a quiet NaN; or fp32), written to
 * out [B, sq, H, D]; if lse is non-NULL also lse[b, h, i] = ln2 * (r_i + log2 l_i), the
 * natural-log log-sum-exp of row i ([CM] Interface table, training output), as a
 * contiguous fp32 [B, H, sq] device array.  Requires run->kv_visited == sk_total
 * and a run not completed by fixedm_attn_fwd_final (FIXEDM_ERR_STATE otherwise); workspace
 * and workspace_bytes as in fixedm_attn_fwd.  Reads the workspace only, so it may be
 * called again. */
fixedm_status fixedm_finalize(const fixedm_bounds_t* bounds, const fixedm_run_t* run,
                              const void* workspace, size_t workspace_bytes,
                              fixedm_tensor out, int32_t out_dtype,
                              float* lse, void* stream);

/* Static string naming a status code. */
const char* fixedm_status_string(fixedm_status s);

#ifdef __cplusplus
}
#endif

#endif /* FIXEDM_H */
