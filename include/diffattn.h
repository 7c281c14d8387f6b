/*
 * diffattn.h -- C ABI of the MI355X (gfx950) differential-attention library.
 *
 * The library computes differential attention -- prefill and decode forward
 * passes, the training backward of V1 (through its norm) and V2, and the two
 * projections on either side of the V2 attention -- as described on two web
 * pages:
 *   [P1] "Differential Transformer | ICLR 2025 Oral" (dainus.ai blog),
 *        sections "Differential Attention: 빼기의 힘", "λ의 역할과 학습",
 *        "파라미터 효율성";
 *   [P2] "Differential Transformer V2" (pogovet.com summary), 상세 정리 §1-§4, §7.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Return value: DIFFATTN_OK (0) on success, a negative DIFFATTN_E_* code on
 *    error.  Nothing throws.  diffattn_last_error() returns a message for the
 *    last nonzero code returned on the calling thread.
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    keeps no pointer after a call returns, allocates nothing and does not
 *    synchronise: work is enqueued asynchronously on `stream`, a hipStream_t
 *    passed as void* (NULL = the default stream).
 *  - Tensors are dense and row-major in the index order given.  Pointers to
 *    bf16/fp32 activation tensors (q, k, v, caches, out) and to workspaces
 *    must be 16-byte aligned; pointers to per-token/per-head scalars
 *    (lambda_logit, norm_weight, cu_seqlens, cache_len) 4-byte aligned
 *    (DIFFATTN_E_ALIGN otherwise).
 *  - Arguments are validated before anything is launched, so a call that
 *    returns an error has not touched any output.  DIFFATTN_E_HIP reports a
 *    failed launch (message from the HIP runtime).
 *  - "bf16" is bfloat16 stored as 16-bit words; "fp32" is IEEE binary32.
 *  - Empty problems (a zero batch or length) return DIFFATTN_OK and launch
 *    nothing, except diffattn_v1_bwd, which still writes its two parameter
 *    gradients (empty sums: zeros).
 */
#ifndef DIFFATTN_H_
#define DIFFATTN_H_

#include <stddef.h>

#if defined(__GNUC__) || defined(__clang__)
#define DIFFATTN_API __attribute__((visibility("default")))
#else
#define DIFFATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DIFFATTN_F32 = 0, DIFFATTN_BF16 = 1 } diffattn_dtype;

enum {
  DIFFATTN_OK = 0,
  DIFFATTN_E_INVALID = -1,     /* bad shape, null pointer, non-finite scalar */
  DIFFATTN_E_UNSUPPORTED = -2, /* well-formed, but not a shape/dtype this library runs */
  DIFFATTN_E_ALIGN = -3,       /* a pointer is not 16-byte aligned */
  DIFFATTN_E_WORKSPACE = -4,   /* workspace missing or smaller than the query says */
  DIFFATTN_E_HIP = -5          /* the HIP runtime reported an error at launch */
};

/*
 * V1 differential attention forward (prefill) [P1 "Differential Attention:
 * 빼기의 힘"; norm and factor: P2 §1].  For every batch b, head h and query row i:
 *
 *   P1 = softmax_j(q1_i . k1_j / sqrt(d)),  P2 = softmax_j(q2_i . k2_j / sqrt(d)),
 *   z_i = sum_j (P1_ij - lambda * P2_ij) v_j,
 *   y_i = (1 - lambda_init) * w * z_i / sqrt(mean_c(z_ic^2) + eps),
 *
 * with j <= i when causal != 0 and j over all T keys otherwise.  The mean runs
 * over the dv value channels of the (row, head); w = norm_weight (NULL = ones).
 *
 *   q1, k1, q2, k2 : [B, T, H, d]   in_dtype
 *   v              : [B, T, H, dv]  in_dtype (the pages' V1 uses dv = 2d)
 *   norm_weight    : [dv] fp32 or NULL
 *   out            : [B, T, H, dv] fp32
 *   lambda         : any finite value (the pages allow lambda > 1)
 *   lambda_init    : the layer's initial lambda (see diffattn_lambda_init)
 *   eps            : finite, >= 0
 *   workspace      : device scratch of at least diffattn_v1_workspace_bytes()
 *                    bytes (may be NULL when that is 0); caller-owned, its
 *                    contents on entry are ignored and on exit unspecified.
 *
 * Supported: in_dtype DIFFATTN_F32 with d in 16..128 and dv in 16..256, both
 * multiples of 16; in_dtype DIFFATTN_BF16 with (d, dv) = (128, 256) or
 * (64, 128).  The bf16 path forms P.V in fp16 (11-bit significand), so V
 * entries must lie within the fp16 range (|v| <= 65504; the largest bf16
 * value inside it is 65280).  Larger entries are not supported: they become
 * inf in the fp16 operand and the output is then not finite.
 */
DIFFATTN_API int diffattn_v1_fwd(const void* q1, const void* k1, const void* q2, const void* k2,
                    const void* v, const float* norm_weight, float* out, int B, int T, int H,
                    int d, int dv, float lambda, float lambda_init, float eps, int causal,
                    diffattn_dtype in_dtype, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Workspace bytes diffattn_v1_fwd needs for these sizes (0 for fp32 inputs).
 * Returns 0 for sizes the call would reject. */
DIFFATTN_API size_t diffattn_v1_workspace_bytes(int B, int T, int H, int d, int dv, diffattn_dtype in_dtype);

/*
 * V1 forward for training: diffattn_v1_fwd (bf16 inputs) that also writes
 * what diffattn_v1_bwd needs from the forward:
 *
 *   o1, o2 : [B, T, H, dv] fp32, the normalised per-map outputs
 *            O_k[i] = sum_j P_k,ij v_j (so z = o1 - lambda * o2)
 *   lse    : [B, T, H, 2] fp32, natural-log log-sum-exp of each map's scaled
 *            scores, map 1 first (P_k,ij = exp(q_k,i . k_k,j / sqrt(d) - lse))
 *
 * Other arguments, the workspace and the supported shapes are those of
 * diffattn_v1_fwd with in_dtype DIFFATTN_BF16 (DIFFATTN_F32 is rejected with
 * DIFFATTN_E_UNSUPPORTED).  o1, o2 and lse are caller-owned and 16-byte aligned.
 */
DIFFATTN_API int diffattn_v1_fwd_train(const void* q1, const void* k1, const void* q2,
                          const void* k2, const void* v, const float* norm_weight, float* out,
                          float* o1, float* o2, float* lse, int B, int T, int H, int d, int dv,
                          float lambda, float lambda_init, float eps, int causal,
                          diffattn_dtype in_dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * V1 backward [P1 "Differential Attention: 빼기의 힘"; norm and factor: P2 §1].
 * The pages give the forward only; this is the chain rule through it.  For
 * the loss L = sum(dy * y), with s = 1 - lambda_init, r_i = sqrt(mean(z_i^2) +
 * eps) and g_i = s * w * dy_i:
 *
 *   dz_i = g_i / r_i - z_i <g_i, z_i> / (dv r_i^3),
 *   dnorm_weight = sum_i s dy_i z_i / r_i,   dlambda = -sum_i <dz_i, O2_i>,
 *   map 1 with dO1 = dz and map 2 with dO2 = -lambda dz, each:
 *     P = softmax rows (recomputed from lse), dP = dO V^T,
 *     dS = P o (dP - rowsum(dO o O)),
 *     dq_k = dS K_k / sqrt(d),  dk_k = dS^T Q_k / sqrt(d),
 *   dv = (P1 - lambda P2)^T dz.
 * Sums over i run over every batch, row and head.
 *
 *   q1, k1, q2, k2, v, norm_weight : as diffattn_v1_fwd (bf16)
 *   o1, o2, lse        : from diffattn_v1_fwd_train on the same inputs
 *   dy                 : [B, T, H, dv] fp32, dL/dy
 *   dq1, dk1, dq2, dk2 : [B, T, H, d] fp32 (written)
 *   dv_out             : [B, T, H, dv] fp32 (written)
 *   dlambda            : [1] fp32 (written)
 *   dnorm_weight       : [dv] fp32 (written; the gradient of the norm weight,
 *                        also when norm_weight is NULL, i.e. all ones)
 *   workspace          : device scratch of at least diffattn_v1_bwd_workspace_bytes()
 *                        bytes (may be NULL when that is 0); caller-owned.
 * All reductions run in a fixed order: results are deterministic.  With no
 * rows (B, T or H zero) only dlambda and dnorm_weight are written, as zeros;
 * the other tensor pointers are then not read and may be NULL.
 * Supported: in_dtype DIFFATTN_BF16 with (d, dv) = (128, 256) or (64, 128).
 */
DIFFATTN_API int diffattn_v1_bwd(const void* q1, const void* k1, const void* q2, const void* k2,
                    const void* v, const float* norm_weight, const float* o1, const float* o2,
                    const float* lse, const float* dy, float* dq1, float* dk1, float* dq2,
                    float* dk2, float* dv_out, float* dlambda, float* dnorm_weight, int B,
                    int T, int H, int d, int dv, float lambda, float lambda_init, float eps,
                    int causal, diffattn_dtype in_dtype, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Workspace bytes diffattn_v1_bwd needs (0 for sizes it would reject or with no rows). */
DIFFATTN_API size_t diffattn_v1_bwd_workspace_bytes(int B, int T, int H, int d, int dv);

/*
 * V2 differential attention forward (prefill) [P2 §1, §4].  Hq = 2h query heads
 * attend over Hkv shared key/value heads; query head j reads KV head
 * j / (Hq / Hkv).  For every sequence, query row i and pair p:
 *
 *   O_j[i]   = sum_t softmax_t(q_{i,j} . k_{t,kv(j)} * scale) v_{t,kv(j)},
 *   out[i,p] = O_{2p}[i] - sigmoid(lambda_logit[i,p]) * O_{2p+1}[i],
 *
 * with t <= i when causal != 0.  No norm or scale follows (P2 §4).  Both heads
 * of a pair must sit in one GQA group, so Hq / Hkv must be even (P2 §1).
 *
 * Padded batch (cu_seqlens == NULL): sequences of length T,
 *   q : [B, T, Hq, d] bf16;  k, v : [B, T, Hkv, d] bf16;
 *   lambda_logit : [B, T, Hq/2] fp32;  out : [B, T, Hq/2, d] bf16.
 *   nseq and max_seqlen are ignored.
 * Packed batch (cu_seqlens != NULL): nseq sequences; sequence s owns tokens
 *   cu_seqlens[s] .. cu_seqlens[s+1]-1 of the packed tensors and attends only
 *   within itself.  cu_seqlens is a DEVICE int32 array [nseq + 1], non-
 *   decreasing, starting at 0.  Shapes as above with [B, T] replaced by
 *   [N total tokens]; B is ignored and T is N = cu_seqlens[nseq] (it sizes the
 *   launch), or 0 when the caller does not know N (then nseq * max_seqlen
 *   bounds the tokens).  max_seqlen must be >= every sequence length: it also
 *   sizes the launch (one workgroup row per sequence when every sequence fits
 *   one query tile).
 *
 *   scale : softmax scale; <= 0 selects 1/sqrt(d).
 * Supported: dtype DIFFATTN_BF16, d in {64, 128}.
 */
DIFFATTN_API int diffattn_v2_fwd(const void* q, const void* k, const void* v, const float* lambda_logit,
                    void* out, const int* cu_seqlens, int nseq, int max_seqlen, int B, int T,
                    int Hq, int Hkv, int d, float scale, int causal, diffattn_dtype dtype,
                    void* stream);

/*
 * Grouped differential attention forward (prefill) [P1 "같은 문제, 다른 접근":
 * the follow-up that splits heads into signal and noise heads at 3:1 or 4:1].
 * The page gives the ratio only; the rule here is this reading of it, the V2
 * subtraction with one noise head serving a block of `ratio` signal heads:
 * query heads come in blocks of ratio + 1 inside a GQA group, heads
 * (ratio + 1) m .. (ratio + 1) m + ratio - 1 are the signal heads of block m
 * and head (ratio + 1) m + ratio its noise head.  Output head s (block
 * m = s / ratio, position r = s % ratio) is
 *
 *   out[i,s] = O_{(ratio+1) m + r}[i] - sigmoid(lambda_logit[i,s]) * O_{(ratio+1) m + ratio}[i],
 *
 * with O_j as in diffattn_v2_fwd.  ratio == 1 is diffattn_v2_fwd exactly.
 * Hs = Hq / (ratio + 1) * ratio output heads; lambda_logit is [.., Hs] fp32
 * and out [.., Hs, d] bf16; q, k, v, cu_seqlens, nseq, max_seqlen, B, T, scale,
 * causal and dtype as diffattn_v2_fwd.  Hq / Hkv must be a multiple of
 * ratio + 1 (a block never spans two KV heads); ratio in 1..15.  With ratio
 * 3 or 7 and Hq / Hkv a multiple of 4 (ratio 3) or 8 (ratio 7), every query
 * head is attended once and the noise head is shared through on-chip memory;
 * for other ratios each signal head's workgroup recomputes its block's noise
 * head (2 Hs head-passes instead of Hq).
 */
DIFFATTN_API int diffattn_gda_fwd(const void* q, const void* k, const void* v,
                                  const float* lambda_logit, void* out, const int* cu_seqlens,
                                  int nseq, int max_seqlen, int B, int T, int Hq, int Hkv, int d,
                                  int ratio, float scale, int causal, diffattn_dtype dtype,
                                  void* stream);

/*
 * V2 training forward (padded batches) [P2 §1, §4]: diffattn_v2_fwd's output,
 * plus what diffattn_v2_bwd needs from the forward:
 *
 *   out          : [B, T, Hq/2, d] bf16, as diffattn_v2_fwd
 *   o_heads      : [B, T, Hq, d] bf16, O_j of every query head before the pair
 *                  subtraction
 *   lse          : [B, T, Hq] fp32, log sum_t exp(q_{i,j} . k_{t,kv(j)} * scale)
 *                  over the visible keys (natural log)
 *
 * Other arguments, layouts and support as diffattn_v2_fwd with cu_seqlens ==
 * NULL.  (For speed the kernel rounds q * scale * log2(e) to bf16 before the
 * score product; lse and o_heads carry that rounding.)
 */
DIFFATTN_API int diffattn_v2_fwd_train(const void* q, const void* k, const void* v,
                          const float* lambda_logit, void* out, void* o_heads, float* lse, int B,
                          int T, int Hq, int Hkv, int d, float scale, int causal,
                          diffattn_dtype dtype, void* stream);

/*
 * V2 backward (padded batches).  The pages give the forward [P2 §1, §4] and
 * quote its training throughput, but no gradient; this is the chain rule
 * through that forward.  For the loss L = sum(dout * out), with s =
 * sigmoid(lambda_logit):
 *
 *   dO_2p = dout_p,  dO_2p+1 = -s * dout_p,
 *   dlambda_logit[i,p] = -s (1 - s) <dout[i,p], O_2p+1[i]>,
 *   per query head j: P = softmax rows (recomputed from lse), dP = dO_j V^T,
 *     dS = P o (dP - rowsum(dO_j o O_j)), dq_j = scale dS K,
 *     dk_kv(j) += scale dS^T q_j,  dv_kv(j) += P^T dO_j.
 *
 *   q, k, v, lambda_logit : as diffattn_v2_fwd (padded)
 *   o_heads, lse          : from diffattn_v2_fwd_train on the same inputs
 *   dout                  : [B, T, Hq/2, d] bf16, dL/dout
 *   dq                    : [B, T, Hq, d] fp32 (written)
 *   dk, dv                : [B, T, Hkv, d] fp32 (written; the query heads of a
 *                           GQA group are summed)
 *   dlambda_logit         : [B, T, Hq/2] fp32 (written)
 *   workspace             : device scratch of at least
 *                           diffattn_v2_bwd_workspace_bytes() bytes; caller-owned.
 * Supported: dtype DIFFATTN_BF16, d in {64, 128}, Hq / Hkv even.
 */
DIFFATTN_API int diffattn_v2_bwd(const void* q, const void* k, const void* v,
                    const float* lambda_logit, const void* o_heads, const float* lse,
                    const void* dout, float* dq, float* dk, float* dv, float* dlambda_logit,
                    void* workspace, size_t workspace_bytes, int B, int T, int Hq, int Hkv, int d,
                    float scale, int causal, diffattn_dtype dtype, void* stream);

/* Workspace bytes diffattn_v2_bwd needs (0 for sizes it would reject). */
DIFFATTN_API size_t diffattn_v2_bwd_workspace_bytes(int B, int T, int Hq, int Hkv, int d);

/*
 * V2 training forward and backward of packed (varlen) batches: as
 * diffattn_v2_fwd_train and diffattn_v2_bwd, with the tensors packed [N, ...]
 * and sequence s owning tokens cu_seqlens[s] .. cu_seqlens[s+1]-1 (attention
 * never crosses a sequence), as in diffattn_v2_fwd's packed form.
 *
 *   cu_seqlens : device int32 [nseq + 1], cu_seqlens[0] = 0, non-decreasing,
 *                cu_seqlens[nseq] = N (not checked: it lives on the device);
 *                every token's gradients are written once by its sequence
 *   max_seqlen : the longest sequence (forward only; an upper bound is fine)
 *   N          : the packed token count cu_seqlens[nseq] (sizes the launches)
 *   q, o_heads, dq : [N, Hq, d];  k, v, dk, dv : [N, Hkv, d];
 *   lambda_logit, dlambda_logit : [N, Hq/2];  lse : [N, Hq];  out, dout : [N, Hq/2, d]
 *   workspace  : at least diffattn_v2_varlen_bwd_workspace_bytes(N, nseq, ...)
 *                bytes (per-row values of every sequence padded to 64 rows).
 * Supported shapes and dtypes as for the padded calls.  N = 0 or nseq = 0 is
 * a no-op.
 */
DIFFATTN_API int diffattn_v2_varlen_fwd_train(const void* q, const void* k, const void* v,
                                 const float* lambda_logit, const int* cu_seqlens, int nseq,
                                 int max_seqlen, long long N, void* out, void* o_heads,
                                 float* lse, int Hq, int Hkv, int d, float scale, int causal,
                                 diffattn_dtype dtype, void* stream);
DIFFATTN_API int diffattn_v2_varlen_bwd(const void* q, const void* k, const void* v,
                           const float* lambda_logit, const int* cu_seqlens, int nseq,
                           const void* o_heads, const float* lse, const void* dout, float* dq,
                           float* dk, float* dv, float* dlambda_logit, void* workspace,
                           size_t workspace_bytes, long long N, int Hq, int Hkv, int d,
                           float scale, int causal, diffattn_dtype dtype, void* stream);
DIFFATTN_API size_t diffattn_v2_varlen_bwd_workspace_bytes(long long N, int nseq, int Hq, int Hkv,
                                              int d);

/*
 * V1 decode step [P1 "Differential Attention: 빼기의 힘"; norm and factor: P2
 * §1]: one new query row per (batch entry, head) against the cached K1, K2
 * and V.  The cache already holds the new token; entry b attends to positions
 * 0 .. cache_len[b]-1 (all S_max when cache_len == NULL), lengths clamped to
 * [0, S_max]:
 *
 *   z = sum_k (softmax_k(q1 . k1_k / sqrt(d)) - lambda softmax_k(q2 . k2_k / sqrt(d))) v_k,
 *   y = (1 - lambda_init) * w * z / sqrt(mean_c(z_c^2) + eps).
 *
 * An entry with no cached position gives zeros.
 *
 *   q1, q2            : [B, H, d] bf16
 *   k1_cache, k2_cache: [B, S_max, H, d] bf16
 *   v_cache           : [B, S_max, H, dv] bf16
 *   cache_len         : DEVICE int32 [B] or NULL
 *   norm_weight       : [dv] fp32 or NULL (ones)
 *   out               : [B, H, dv] fp32
 *   workspace         : device scratch of at least diffattn_v1_decode_workspace_bytes()
 *                       bytes for per-slice partial results; caller-owned.
 * Supported: dtype DIFFATTN_BF16, (d, dv) = (128, 256) or (64, 128).
 */
DIFFATTN_API int diffattn_v1_decode(const void* q1, const void* q2, const void* k1_cache,
                       const void* k2_cache, const void* v_cache, const int* cache_len,
                       const float* norm_weight, float* out, void* workspace,
                       size_t workspace_bytes, int B, int S_max, int H, int d, int dv,
                       float lambda, float lambda_init, float eps, diffattn_dtype dtype,
                       void* stream);

/* Workspace bytes diffattn_v1_decode needs (0 for sizes it would reject). */
DIFFATTN_API size_t diffattn_v1_decode_workspace_bytes(int B, int S_max, int H, int d, int dv);

/*
 * V2 decode step [P2 §1, §2]: one new query row per sequence against its KV
 * cache.  The cache already holds the new token's K and V; entry b attends to
 * positions 0 .. cache_len[b]-1 (all S_max when cache_len == NULL).  An entry
 * with no cached position gives zeros; lengths are clamped to [0, S_max].
 *
 *   q            : [B, Hq, d] bf16
 *   k_cache      : [B, S_max, Hkv, d] bf16;  v_cache: same
 *   cache_len    : DEVICE int32 [B] or NULL
 *   lambda_logit : [B, Hq/2] fp32
 *   out          : [B, Hq/2, d] bf16
 *   workspace    : device scratch of at least diffattn_v2_decode_workspace_bytes()
 *                  bytes for per-slice partial results; caller-owned.
 *   scale        : <= 0 selects 1/sqrt(d).
 * Supported: dtype DIFFATTN_BF16, d in {64, 128}, Hq / Hkv even and <= 16.
 */
DIFFATTN_API int diffattn_v2_decode(const void* q, const void* k_cache, const void* v_cache,
                       const int* cache_len, const float* lambda_logit, void* out,
                       void* workspace, size_t workspace_bytes, int B, int S_max, int Hq,
                       int Hkv, int d, float scale, diffattn_dtype dtype, void* stream);

/* Workspace bytes diffattn_v2_decode needs (0 for sizes it would reject). */
DIFFATTN_API size_t diffattn_v2_decode_workspace_bytes(int B, int S_max, int Hq, int Hkv, int d);

/*
 * Grouped differential attention decode step [P1 "같은 문제, 다른 접근"; rule
 * as diffattn_gda_fwd]: diffattn_v2_decode with blocks of `ratio` signal heads
 * and one noise head.  lambda_logit : [B, Hs] fp32; out : [B, Hs, d] bf16 with
 * Hs = Hq / (ratio + 1) * ratio; the other arguments as diffattn_v2_decode.
 * Every query head is attended once, so the noise head is not recomputed.
 * Supported: dtype DIFFATTN_BF16, d in {64, 128}, Hq / Hkv a multiple of
 * ratio + 1 and <= 16, ratio in 1..15.
 */
DIFFATTN_API int diffattn_gda_decode(const void* q, const void* k_cache, const void* v_cache,
                                     const int* cache_len, const float* lambda_logit, void* out,
                                     void* workspace, size_t workspace_bytes, int B, int S_max,
                                     int Hq, int Hkv, int d, int ratio, float scale,
                                     diffattn_dtype dtype, void* stream);

/* Workspace bytes diffattn_gda_decode needs (0 for sizes it would reject). */
DIFFATTN_API size_t diffattn_gda_decode_workspace_bytes(int B, int S_max, int Hq, int Hkv, int d,
                                                        int ratio);

/*
 * diffattn_v2_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and errors as diffattn_v2_decode, minus
 * the workspace: the per-slice partial results go to an array the library
 * owns, DIFFATTN_V2_DECODE_NOALLOC_MAX_BYTES on each GPU it runs on, held
 * until the process ends.  Sizes whose diffattn_v2_decode_workspace_bytes()
 * exceeds that limit are rejected with DIFFATTN_E_UNSUPPORTED (at Hq 64, d 128
 * that is above roughly B = 990 unsplit sequences; a split cache needs at most
 * about 34 KB per workgroup of the launch).  The call allocates nothing (no
 * hipMalloc, no allocating library routine); its first call on a device looks
 * up that device's array.  All calls on one GPU share the array, so calls
 * that overlap on one GPU (different streams, or threads) race: serialise
 * them.  Nothing in the array needs clearing between calls.
 */
#define DIFFATTN_V2_DECODE_NOALLOC_MAX_BYTES ((size_t)32 << 20)
DIFFATTN_API int diffattn_v2_decode_noalloc(const void* q, const void* k_cache,
                                            const void* v_cache, const int* cache_len,
                                            const float* lambda_logit, void* out, int B,
                                            int S_max, int Hq, int Hkv, int d, float scale,
                                            diffattn_dtype dtype, void* stream);

/*
 * V2 coefficient logits [P2 §1]: the coefficient that scales the second
 * head of each pair is projected from the layer input, one per token and
 * pair, and passes through a sigmoid where it is used (diffattn_v2_fwd and
 * diffattn_v2_decode apply it).  This computes the projection:
 *
 *   logits[n, p] = sum_c x[n, c] * w_lambda[p, c]     (fp32 accumulation)
 *
 *   x        : [N, d_model] bf16, the layer input (N tokens)
 *   w_lambda : [h, d_model] bf16, one weight row per pair
 *   logits   : [N, h] fp32 (written), the lambda_logit input of the V2 calls
 *
 * Supported: dtype DIFFATTN_BF16, h in {16, 32, 48, 64}, d_model a multiple of
 * 256.  x and w_lambda 16-byte aligned, logits 4-byte aligned.  N = 0 is a
 * no-op (pointers are then not read).
 */
DIFFATTN_API int diffattn_v2_lambda_proj(const void* x, const void* w_lambda, float* logits,
                            long long N, int d_model, int h, diffattn_dtype dtype,
                            void* stream);

/*
 * Output projection [P2 §1, §7]: after the subtraction each token carries
 * h*d columns, so the projection back to d_model has the baseline's shape
 * (half the input width of a 2h-head model with the same query heads):
 *
 *   y[m, n] = sum_k attn_out[m, k] * w_o[n, k]        (fp32 accumulation)
 *
 *   attn_out : [M, K] bf16 (e.g. the V2 output [tokens, h*d], or V1's z)
 *   w_o      : [N, K] bf16, one weight row per output feature
 *   y        : [M, N] bf16 (written)
 *
 * Supported: dtype DIFFATTN_BF16, K a multiple of 64 (and below 2^24), N a
 * multiple of 4; all pointers 16-byte aligned.  M = 0 is a no-op.
 */
DIFFATTN_API int diffattn_out_proj(const void* attn_out, const void* w_o, void* y, long long M,
                      long long K, long long N, diffattn_dtype dtype, void* stream);

/* Initial lambda of 1-based layer `layer` [P1 "λ의 역할과 학습"]:
 * 0.8 - 0.6 * exp(-0.3 * (layer - 1)) in fp32.  Returns NaN (and sets the last
 * error) for layer < 1. */
DIFFATTN_API float diffattn_lambda_init(int layer);

/* Message for the last nonzero code returned on this thread ("" if none). */
DIFFATTN_API const char* diffattn_last_error(void);

/* Library version as major * 10000 + minor * 100 + patch. */
DIFFATTN_API int diffattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DIFFATTN_H_ */
