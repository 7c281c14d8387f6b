// C ABI of the differential-attention library: argument validation, workspace
// queries and kernel dispatch.  Every check runs before any launch, so an
// error return leaves the outputs untouched.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "../../include/diffattn.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return DIFFATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DIFFATTN_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Product of non-negative ints, or -1 on overflow past int64.
long long prod(std::initializer_list<long long> xs) {
  long long r = 1;
  for (long long x : xs) {
    if (x < 0) return -1;
    if (x != 0 && r > (long long)(INT64_MAX / x)) return -1;
    r *= x;
  }
  return r;
}

// Head-layout and dtype checks shared by the V2 (ratio 1) and grouped
// (ratio r) prefill, training-forward and backward entry points; returns
// DIFFATTN_OK or a failure code.
int v2_heads_check(const char* fn, int Hq, int Hkv, int d, float scale, int causal,
                   diffattn_dtype dtype, int ratio = 1) {
  if (Hq <= 0 || Hkv <= 0 || d <= 0)
    return fail(DIFFATTN_E_INVALID, "%s: bad head sizes Hq=%d Hkv=%d d=%d", fn, Hq, Hkv, d);
  if (ratio < 1 || ratio > 15)
    return fail(DIFFATTN_E_INVALID, "%s: ratio=%d must be in 1..15", fn, ratio);
  if (ratio == 1 && Hq % 2)
    return fail(DIFFATTN_E_INVALID, "%s: Hq=%d must be even (pairs of heads)", fn, Hq);
  if (Hq % Hkv)
    return fail(DIFFATTN_E_INVALID, "%s: Hq=%d must be a multiple of Hkv=%d", fn, Hq, Hkv);
  if (ratio == 1 && (Hq / Hkv) % 2)
    return fail(DIFFATTN_E_INVALID,
                "%s: Hq/Hkv=%d must be even so both heads of a pair share one KV head", fn,
                Hq / Hkv);
  if ((Hq / Hkv) % (ratio + 1))
    return fail(DIFFATTN_E_INVALID,
                "%s: Hq/Hkv=%d must be a multiple of ratio + 1 = %d so every block of signal "
                "heads and its noise head share one KV head", fn, Hq / Hkv, ratio + 1);
  if (causal != 0 && causal != 1) return fail(DIFFATTN_E_INVALID, "%s: causal must be 0 or 1", fn);
  if (!isfinite(scale)) return fail(DIFFATTN_E_INVALID, "%s: scale must be finite", fn);
  if (dtype != DIFFATTN_BF16)
    return fail(dtype == DIFFATTN_F32 ? DIFFATTN_E_UNSUPPORTED : DIFFATTN_E_INVALID,
                "%s: only bf16 is supported", fn);
  if (d != 64 && d != 128) return fail(DIFFATTN_E_UNSUPPORTED, "%s: d=%d not in {64, 128}", fn, d);
  return DIFFATTN_OK;
}

bool v1_shape_supported(int d, int dv, diffattn_dtype dt) {
  if (dt == DIFFATTN_F32) return d >= 16 && d <= 128 && d % 16 == 0 && dv >= 16 && dv <= 256 && dv % 16 == 0;
  if (dt == DIFFATTN_BF16) return (d == 128 && dv == 256) || (d == 64 && dv == 128);
  return false;
}

// Checks shared by the V1 forward and training-forward entry points: sizes,
// dtype, flags, shape support, alignment and workspace; DIFFATTN_OK or a code.
int v1_fwd_check(const char* fn, const void* const* ptrs, int nptrs,
                        const float* norm_weight, int B, int T, int H, int d, int dv,
                        float lambda, float lambda_init, float eps, int causal,
                        diffattn_dtype in_dtype, void* workspace, size_t workspace_bytes) {
  for (int i = 0; i < nptrs; ++i)
    if (!ptrs[i]) return fail(DIFFATTN_E_INVALID, "%s: null tensor pointer", fn);
  if (B < 0 || T < 0 || H < 0 || d <= 0 || dv <= 0)
    return fail(DIFFATTN_E_INVALID, "%s: bad sizes B=%d T=%d H=%d d=%d dv=%d", fn, B, T, H, d, dv);
  if (in_dtype != DIFFATTN_F32 && in_dtype != DIFFATTN_BF16)
    return fail(DIFFATTN_E_INVALID, "%s: unknown dtype %d", fn, (int)in_dtype);
  if (causal != 0 && causal != 1) return fail(DIFFATTN_E_INVALID, "%s: causal must be 0 or 1", fn);
  if (!isfinite(lambda) || !isfinite(lambda_init) || !isfinite(eps) || eps < 0.f)
    return fail(DIFFATTN_E_INVALID, "%s: lambda, lambda_init must be finite and eps finite >= 0", fn);
  if (!v1_shape_supported(d, dv, in_dtype))
    return fail(DIFFATTN_E_UNSUPPORTED,
                "%s: (d=%d, dv=%d) not supported for %s inputs (fp32: multiples of 16, d<=128, "
                "dv<=256; bf16: (128,256) or (64,128))",
                fn, d, dv, in_dtype == DIFFATTN_F32 ? "fp32" : "bf16");
  const long long nout = prod({B, T, H, dv});
  if (nout < 0 || prod({B, T, H, d}) < 0 || nout > (1LL << 40))
    return fail(DIFFATTN_E_INVALID, "%s: problem too large", fn);
  for (int i = 0; i < nptrs; ++i)
    if (!aligned16(ptrs[i]))
      return fail(DIFFATTN_E_ALIGN, "%s: tensor pointers must be 16-byte aligned", fn);
  if (norm_weight && !aligned4(norm_weight))
    return fail(DIFFATTN_E_ALIGN, "%s: norm_weight must be 4-byte aligned", fn);
  if (nout == 0) return DIFFATTN_OK;
  const size_t need = diffattn_v1_workspace_bytes(B, T, H, d, dv, in_dtype);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(DIFFATTN_E_WORKSPACE, "%s: workspace of %zu bytes required (got %zu%s)", fn, need,
                workspace_bytes, workspace ? "" : ", NULL");
  if (need > 0 && !aligned16(workspace))
    return fail(DIFFATTN_E_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  return DIFFATTN_OK;
}

}  // namespace

extern "C" {

int diffattn_version(void) { return 100; }

const char* diffattn_last_error(void) { return g_last_error.c_str(); }

float diffattn_lambda_init(int layer) {
  if (layer < 1) {
    fail(DIFFATTN_E_INVALID, "diffattn_lambda_init: layer must be >= 1 (got %d)", layer);
    return NAN;
  }
  g_last_error.clear();
  return 0.8f - 0.6f * expf(-0.3f * (float)(layer - 1));
}

size_t diffattn_v1_workspace_bytes(int B, int T, int H, int d, int dv, diffattn_dtype in_dtype) {
  if (B < 0 || T < 0 || H < 0 || !v1_shape_supported(d, dv, in_dtype)) return 0;
  if (in_dtype != DIFFATTN_BF16 || prod({B, T, H}) == 0) return 0;
  return diffattn::v1_bf16_workspace_bytes(B, T, H, d, dv);
}

int diffattn_v1_fwd(const void* q1, const void* k1, const void* q2, const void* k2,
                    const void* v, const float* norm_weight, float* out, int B, int T, int H,
                    int d, int dv, float lambda, float lambda_init, float eps, int causal,
                    diffattn_dtype in_dtype, void* workspace, size_t workspace_bytes,
                    void* stream) {
  const char* fn = "diffattn_v1_fwd";
  const void* ptrs[] = {q1, k1, q2, k2, v, out};
  const int rc = v1_fwd_check(fn, ptrs, 6, norm_weight, B, T, H, d, dv, lambda, lambda_init, eps,
                              causal, in_dtype, workspace, workspace_bytes);
  if (rc != DIFFATTN_OK) return rc;
  if (prod({B, T, H}) == 0) return ok();
  diffattn::V1Args a{q1, k1, q2, k2, v, norm_weight, out, B, T, H, d, dv,
                     lambda, lambda_init, eps, causal};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (in_dtype == DIFFATTN_F32) return from_hip(diffattn::launch_v1_f32(a, s), fn);
  return from_hip(diffattn::launch_v1_bf16(a, workspace, s), fn);
}

int diffattn_v1_fwd_train(const void* q1, const void* k1, const void* q2, const void* k2,
                          const void* v, const float* norm_weight, float* out, float* o1,
                          float* o2, float* lse, int B, int T, int H, int d, int dv, float lambda,
                          float lambda_init, float eps, int causal, diffattn_dtype in_dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "diffattn_v1_fwd_train";
  if (in_dtype != DIFFATTN_BF16)
    return fail(in_dtype == DIFFATTN_F32 ? DIFFATTN_E_UNSUPPORTED : DIFFATTN_E_INVALID,
                "%s: only bf16 inputs are supported", fn);
  const void* ptrs[] = {q1, k1, q2, k2, v, out, o1, o2, lse};
  const int rc = v1_fwd_check(fn, ptrs, 9, norm_weight, B, T, H, d, dv, lambda, lambda_init, eps,
                              causal, in_dtype, workspace, workspace_bytes);
  if (rc != DIFFATTN_OK) return rc;
  if (prod({B, T, H}) == 0) return ok();
  diffattn::V1Args a{q1, k1, q2, k2, v, norm_weight, out, B, T, H, d, dv,
                     lambda, lambda_init, eps, causal, o1, o2, lse};
  return from_hip(diffattn::launch_v1_bf16(a, workspace, static_cast<hipStream_t>(stream)), fn);
}

size_t diffattn_v1_bwd_workspace_bytes(int B, int T, int H, int d, int dv) {
  if (B < 0 || T < 0 || H < 0 || !v1_shape_supported(d, dv, DIFFATTN_BF16)) return 0;
  if (prod({B, T, H, dv}) <= 0) return 0;
  return diffattn::v1_bwd_workspace_bytes(B, T, H, d, dv);
}

int diffattn_v1_bwd(const void* q1, const void* k1, const void* q2, const void* k2,
                    const void* v, const float* norm_weight, const float* o1, const float* o2,
                    const float* lse, const float* dy, float* dq1, float* dk1, float* dq2,
                    float* dk2, float* dv_out, float* dlambda, float* dnorm_weight, int B, int T,
                    int H, int d, int dv, float lambda, float lambda_init, float eps, int causal,
                    diffattn_dtype in_dtype, void* workspace, size_t workspace_bytes,
                    void* stream) {
  const char* fn = "diffattn_v1_bwd";
  if (in_dtype != DIFFATTN_BF16)
    return fail(in_dtype == DIFFATTN_F32 ? DIFFATTN_E_UNSUPPORTED : DIFFATTN_E_INVALID,
                "%s: only bf16 inputs are supported", fn);
  if (!dlambda || !dnorm_weight) return fail(DIFFATTN_E_INVALID, "%s: null dlambda or dnorm_weight", fn);
  if (B < 0 || T < 0 || H < 0 || d <= 0 || dv <= 0)
    return fail(DIFFATTN_E_INVALID, "%s: bad sizes B=%d T=%d H=%d d=%d dv=%d", fn, B, T, H, d, dv);
  if (causal != 0 && causal != 1) return fail(DIFFATTN_E_INVALID, "%s: causal must be 0 or 1", fn);
  if (!isfinite(lambda) || !isfinite(lambda_init) || !isfinite(eps) || eps < 0.f)
    return fail(DIFFATTN_E_INVALID, "%s: lambda, lambda_init must be finite and eps finite >= 0", fn);
  if (!v1_shape_supported(d, dv, in_dtype))
    return fail(DIFFATTN_E_UNSUPPORTED, "%s: (d=%d, dv=%d) not in {(128, 256), (64, 128)}", fn, d,
                dv);
  const long long nout = prod({B, T, H, dv});
  if (nout < 0 || nout > (1LL << 40)) return fail(DIFFATTN_E_INVALID, "%s: problem too large", fn);
  // with no rows the tensors are not read: only dlambda and dnorm_weight must be valid
  const void* ptrs[] = {q1, k1, q2, k2, v, o1, o2, dy, dq1, dk1, dq2, dk2, dv_out};
  if (nout != 0) {
    for (const void* p : ptrs)
      if (!p) return fail(DIFFATTN_E_INVALID, "%s: null tensor pointer", fn);
    if (!lse) return fail(DIFFATTN_E_INVALID, "%s: null lse", fn);
    for (const void* p : ptrs)
      if (!aligned16(p))
        return fail(DIFFATTN_E_ALIGN, "%s: tensor pointers must be 16-byte aligned", fn);
  }
  if (!aligned4(lse) || !aligned4(dlambda) || !aligned4(dnorm_weight) ||
      (norm_weight && !aligned4(norm_weight)))
    return fail(DIFFATTN_E_ALIGN, "%s: lse, norm_weight, dlambda and dnorm_weight must be 4-byte aligned", fn);
  // with no rows only the parameter gradients (sums over nothing) are written
  const size_t need = diffattn_v1_bwd_workspace_bytes(B, T, H, d, dv);
  if (nout != 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(DIFFATTN_E_WORKSPACE, "%s: workspace of %zu bytes required (got %zu%s)", fn, need,
                workspace_bytes, workspace ? "" : ", NULL");
  if (nout != 0 && !aligned16(workspace))
    return fail(DIFFATTN_E_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  diffattn::V1BwdArgs a{};
  a.q1 = static_cast<const uint16_t*>(q1);
  a.k1 = static_cast<const uint16_t*>(k1);
  a.q2 = static_cast<const uint16_t*>(q2);
  a.k2 = static_cast<const uint16_t*>(k2);
  a.v = static_cast<const uint16_t*>(v);
  a.norm_weight = norm_weight;
  a.o1 = o1;
  a.o2 = o2;
  a.lse = lse;
  a.dy = dy;
  a.dq1 = dq1;
  a.dk1 = dk1;
  a.dq2 = dq2;
  a.dk2 = dk2;
  a.dvg = dv_out;
  a.dlambda = dlambda;
  a.dnorm_weight = dnorm_weight;
  a.workspace = workspace;
  a.B = B;
  a.T = T;
  a.H = H;
  a.d = d;
  a.dv = dv;
  a.lambda = lambda;
  a.lambda_init = lambda_init;
  a.eps = eps;
  a.causal = causal;
  return from_hip(diffattn::launch_v1_backward(a, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"

namespace {

// The V2 (ratio 1) and grouped (ratio r) prefill: checks, then one launch.
int prefill_call(const char* fn, const void* q, const void* k, const void* v,
                 const float* lambda_logit, void* out, const int* cu_seqlens, int nseq,
                 int max_seqlen, int B, int T, int Hq, int Hkv, int d, int ratio, float scale,
                 int causal, diffattn_dtype dtype, void* stream) {
  if (!q || !k || !v || !lambda_logit || !out)
    return fail(DIFFATTN_E_INVALID, "%s: null tensor pointer", fn);
  const int rc = v2_heads_check(fn, Hq, Hkv, d, scale, causal, dtype, ratio);
  if (rc != DIFFATTN_OK) return rc;
  int nseq_eff, maxlen;
  if (cu_seqlens) {
    if (nseq < 0 || max_seqlen < 0 || T < 0)
      return fail(DIFFATTN_E_INVALID, "%s: nseq=%d max_seqlen=%d T=%d must be >= 0", fn, nseq,
                  max_seqlen, T);
    if (prod({T, Hq, d}) > (1LL << 40)) return fail(DIFFATTN_E_INVALID, "%s: problem too large", fn);
    nseq_eff = nseq;
    maxlen = max_seqlen;
  } else {
    if (B < 0 || T < 0) return fail(DIFFATTN_E_INVALID, "%s: B=%d T=%d must be >= 0", fn, B, T);
    if (prod({B, T, Hq, d}) > (1LL << 40)) return fail(DIFFATTN_E_INVALID, "%s: problem too large", fn);
    nseq_eff = B;
    maxlen = T;
  }
  const void* ptrs[] = {q, k, v, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(DIFFATTN_E_ALIGN, "%s: tensor pointers must be 16-byte aligned", fn);
  if (!aligned4(lambda_logit) || (cu_seqlens && !aligned4(cu_seqlens)))
    return fail(DIFFATTN_E_ALIGN, "%s: lambda_logit and cu_seqlens must be 4-byte aligned", fn);
  if (nseq_eff == 0 || maxlen == 0) return ok();
  diffattn::V2Args a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.logit = lambda_logit;
  a.out = static_cast<uint16_t*>(out);
  a.cu_seqlens = cu_seqlens;
  a.nseq = nseq_eff;
  a.max_seqlen = maxlen;
  a.T = T;
  a.N = (cu_seqlens && T > 0) ? (long long)T : -1;  // packed: T is the token count, if known
  a.Hq = Hq;
  a.ratio = ratio;
  a.nout = Hq / (ratio + 1) * ratio;
  a.Hkv = Hkv;
  a.d = d;
  a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
  a.causal = causal;
  return from_hip(diffattn::launch_v2_prefill(a, static_cast<hipStream_t>(stream)), fn);
}

}  // namespace

extern "C" {

int diffattn_v2_fwd(const void* q, const void* k, const void* v, const float* lambda_logit,
                    void* out, const int* cu_seqlens, int nseq, int max_seqlen, int B, int T,
                    int Hq, int Hkv, int d, float scale, int causal, diffattn_dtype dtype,
                    void* stream) {
  return prefill_call("diffattn_v2_fwd", q, k, v, lambda_logit, out, cu_seqlens, nseq,
                      max_seqlen, B, T, Hq, Hkv, d, 1, scale, causal, dtype, stream);
}

int diffattn_gda_fwd(const void* q, const void* k, const void* v, const float* lambda_logit,
                     void* out, const int* cu_seqlens, int nseq, int max_seqlen, int B, int T,
                     int Hq, int Hkv, int d, int ratio, float scale, int causal,
                     diffattn_dtype dtype, void* stream) {
  return prefill_call("diffattn_gda_fwd", q, k, v, lambda_logit, out, cu_seqlens, nseq,
                      max_seqlen, B, T, Hq, Hkv, d, ratio, scale, causal, dtype, stream);
}

int diffattn_v2_fwd_train(const void* q, const void* k, const void* v, const float* lambda_logit,
                          void* out, void* o_heads, float* lse, int B, int T, int Hq, int Hkv,
                          int d, float scale, int causal, diffattn_dtype dtype, void* stream) {
  const char* fn = "diffattn_v2_fwd_train";
  if (!q || !k || !v || !lambda_logit || !out || !o_heads || !lse)
    return fail(DIFFATTN_E_INVALID, "%s: null tensor pointer", fn);
  const int rc = v2_heads_check(fn, Hq, Hkv, d, scale, causal, dtype);
  if (rc != DIFFATTN_OK) return rc;
  if (B < 0 || T < 0) return fail(DIFFATTN_E_INVALID, "%s: B=%d T=%d must be >= 0", fn, B, T);
  if (prod({B, T, Hq, d}) > (1LL << 40)) return fail(DIFFATTN_E_INVALID, "%s: problem too large", fn);
  const void* ptrs[] = {q, k, v, out, o_heads};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(DIFFATTN_E_ALIGN, "%s: tensor pointers must be 16-byte aligned", fn);
  if (!aligned4(lambda_logit) || !aligned4(lse))
    return fail(DIFFATTN_E_ALIGN, "%s: lambda_logit and lse must be 4-byte aligned", fn);
  if (B == 0 || T == 0) return ok();
  diffattn::V2Args a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.logit = lambda_logit;
  a.out = static_cast<uint16_t*>(out);
  a.cu_seqlens = nullptr;
  a.nseq = B;
  a.max_seqlen = T;
  a.T = T;
  a.N = -1;
  a.Hq = Hq;
  a.nout = Hq / 2;
  a.Hkv = Hkv;
  a.d = d;
  a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
  a.causal = causal;
  a.o_heads = static_cast<uint16_t*>(o_heads);
  a.lse = lse;
  return from_hip(diffattn::launch_v2_prefill(a, static_cast<hipStream_t>(stream)), fn);
}

size_t diffattn_v2_bwd_workspace_bytes(int B, int T, int Hq, int Hkv, int d) {
  if (B < 0 || T < 0 || Hq <= 0 || Hkv <= 0 || Hq % 2 || Hq % Hkv || (Hq / Hkv) % 2) return 0;
  if (d != 64 && d != 128) return 0;
  if (prod({B, T, Hq, d}) < 0) return 0;
  return diffattn::v2_bwd_workspace_bytes(B, T, Hq);
}

int diffattn_v2_bwd(const void* q, const void* k, const void* v, const float* lambda_logit,
                    const void* o_heads, const float* lse, const void* dout, float* dq, float* dk,
                    float* dv, float* dlambda_logit, void* workspace, size_t workspace_bytes,
                    int B, int T, int Hq, int Hkv, int d, float scale, int causal,
                    diffattn_dtype dtype, void* stream) {
  const char* fn = "diffattn_v2_bwd";
  if (!q || !k || !v || !lambda_logit || !o_heads || !lse || !dout || !dq || !dk || !dv ||
      !dlambda_logit)
    return fail(DIFFATTN_E_INVALID, "%s: null tensor pointer", fn);
  const int rc = v2_heads_check(fn, Hq, Hkv, d, scale, causal, dtype);
  if (rc != DIFFATTN_OK) return rc;
  if (B < 0 || T < 0) return fail(DIFFATTN_E_INVALID, "%s: B=%d T=%d must be >= 0", fn, B, T);
  if (prod({B, T, Hq, d}) > (1LL << 40)) return fail(DIFFATTN_E_INVALID, "%s: problem too large", fn);
  const void* ptrs[] = {q, k, v, o_heads, dout, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(DIFFATTN_E_ALIGN, "%s: tensor pointers must be 16-byte aligned", fn);
  if (!aligned4(lambda_logit) || !aligned4(lse) || !aligned4(dlambda_logit))
    return fail(DIFFATTN_E_ALIGN, "%s: lambda_logit, lse and dlambda_logit must be 4-byte aligned", fn);
  if (B == 0 || T == 0) return ok();
  const size_t need = diffattn_v2_bwd_workspace_bytes(B, T, Hq, Hkv, d);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(DIFFATTN_E_WORKSPACE, "%s: workspace of %zu bytes required (got %zu%s)", fn, need,
                workspace_bytes, workspace ? "" : ", NULL");
  if (!aligned16(workspace)) return fail(DIFFATTN_E_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  diffattn::V2BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.logit = lambda_logit;
  a.o_heads = static_cast<const uint16_t*>(o_heads);
  a.lse = lse;
  a.dout = static_cast<const uint16_t*>(dout);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dlogit = dlambda_logit;
  a.delta = static_cast<float*>(workspace);
  a.B = B;
  a.T = T;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
  a.causal = causal;
  a.cu_seqlens = nullptr;
  a.nseq = B;
  a.N = (long long)B * T;
  a.Np = diffattn::v2_bwd_rows(B, T);
  return from_hip(diffattn::launch_v2_backward(a, static_cast<hipStream_t>(stream)), fn);
}

int diffattn_v2_varlen_fwd_train(const void* q, const void* k, const void* v,
                                 const float* lambda_logit, const int* cu_seqlens, int nseq,
                                 int max_seqlen, long long N, void* out, void* o_heads, float* lse,
                                 int Hq, int Hkv, int d, float scale, int causal,
                                 diffattn_dtype dtype, void* stream) {
  const char* fn = "diffattn_v2_varlen_fwd_train";
  if (!q || !k || !v || !lambda_logit || !out || !o_heads || !lse || !cu_seqlens)
    return fail(DIFFATTN_E_INVALID, "%s: null tensor pointer", fn);
  const int rc = v2_heads_check(fn, Hq, Hkv, d, scale, causal, dtype);
  if (rc != DIFFATTN_OK) return rc;
  if (nseq < 0 || max_seqlen < 0 || N < 0)
    return fail(DIFFATTN_E_INVALID, "%s: nseq=%d max_seqlen=%d N=%lld must be >= 0", fn, nseq,
                max_seqlen, N);
  if (prod({N, Hq, d}) > (1LL << 40)) return fail(DIFFATTN_E_INVALID, "%s: problem too large", fn);
  const void* ptrs[] = {q, k, v, out, o_heads};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(DIFFATTN_E_ALIGN, "%s: tensor pointers must be 16-byte aligned", fn);
  if (!aligned4(lambda_logit) || !aligned4(lse) || !aligned4(cu_seqlens))
    return fail(DIFFATTN_E_ALIGN, "%s: lambda_logit, lse and cu_seqlens must be 4-byte aligned", fn);
  if (nseq == 0 || max_seqlen == 0 || N == 0) return ok();
  diffattn::V2Args a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.logit = lambda_logit;
  a.out = static_cast<uint16_t*>(out);
  a.cu_seqlens = cu_seqlens;
  a.nseq = nseq;
  a.max_seqlen = max_seqlen;
  a.T = 0;
  a.N = N;
  a.Hq = Hq;
  a.nout = Hq / 2;
  a.Hkv = Hkv;
  a.d = d;
  a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
  a.causal = causal;
  a.o_heads = static_cast<uint16_t*>(o_heads);
  a.lse = lse;
  return from_hip(diffattn::launch_v2_prefill(a, static_cast<hipStream_t>(stream)), fn);
}

size_t diffattn_v2_varlen_bwd_workspace_bytes(long long N, int nseq, int Hq, int Hkv, int d) {
  if (N < 0 || nseq < 0 || Hq <= 0 || Hkv <= 0 || Hq % 2 || Hq % Hkv || (Hq / Hkv) % 2) return 0;
  if (d != 64 && d != 128) return 0;
  if (prod({N, Hq, d}) < 0 || prod({N, Hq, d}) > (1LL << 40)) return 0;
  if (N == 0 || nseq == 0) return 0;
  return diffattn::v2_bwd_workspace_bytes_rows(diffattn::v2_bwd_varlen_rows(N, nseq), Hq);
}

int diffattn_v2_varlen_bwd(const void* q, const void* k, const void* v, const float* lambda_logit,
                           const int* cu_seqlens, int nseq, const void* o_heads, const float* lse,
                           const void* dout, float* dq, float* dk, float* dv,
                           float* dlambda_logit, void* workspace, size_t workspace_bytes,
                           long long N, int Hq, int Hkv, int d, float scale, int causal,
                           diffattn_dtype dtype, void* stream) {
  const char* fn = "diffattn_v2_varlen_bwd";
  const int rc = v2_heads_check(fn, Hq, Hkv, d, scale, causal, dtype);
  if (rc != DIFFATTN_OK) return rc;
  if (N < 0 || nseq < 0) return fail(DIFFATTN_E_INVALID, "%s: N=%lld nseq=%d must be >= 0", fn, N, nseq);
  if (prod({N, Hq, d}) > (1LL << 40)) return fail(DIFFATTN_E_INVALID, "%s: problem too large", fn);
  if (N == 0 || nseq == 0) return ok();
  if (!q || !k || !v || !lambda_logit || !cu_seqlens || !o_heads || !lse || !dout || !dq || !dk ||
      !dv || !dlambda_logit)
    return fail(DIFFATTN_E_INVALID, "%s: null tensor pointer", fn);
  const void* ptrs[] = {q, k, v, o_heads, dout, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(DIFFATTN_E_ALIGN, "%s: tensor pointers must be 16-byte aligned", fn);
  if (!aligned4(lambda_logit) || !aligned4(lse) || !aligned4(dlambda_logit) || !aligned4(cu_seqlens))
    return fail(DIFFATTN_E_ALIGN, "%s: lambda_logit, lse, dlambda_logit and cu_seqlens must be 4-byte aligned", fn);
  const size_t need = diffattn_v2_varlen_bwd_workspace_bytes(N, nseq, Hq, Hkv, d);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(DIFFATTN_E_WORKSPACE, "%s: workspace of %zu bytes required (got %zu%s)", fn, need,
                workspace_bytes, workspace ? "" : ", NULL");
  if (!aligned16(workspace)) return fail(DIFFATTN_E_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  diffattn::V2BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.logit = lambda_logit;
  a.o_heads = static_cast<const uint16_t*>(o_heads);
  a.lse = lse;
  a.dout = static_cast<const uint16_t*>(dout);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dlogit = dlambda_logit;
  a.delta = static_cast<float*>(workspace);
  a.B = 0;
  a.T = 0;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
  a.causal = causal;
  a.cu_seqlens = cu_seqlens;
  a.nseq = nseq;
  a.N = N;
  a.Np = diffattn::v2_bwd_varlen_rows(N, nseq);
  return from_hip(diffattn::launch_v2_backward(a, static_cast<hipStream_t>(stream)), fn);
}

size_t diffattn_v1_decode_workspace_bytes(int B, int S_max, int H, int d, int dv) {
  if (B < 0 || S_max < 0 || H <= 0) return 0;
  if (!((d == 128 && dv == 256) || (d == 64 && dv == 128))) return 0;
  int split_len, nsplit;
  diffattn::v1_decode_split(B, S_max, H, &split_len, &nsplit);
  const long long n = prod({B, H, 2, nsplit, dv + 4});
  return n < 0 ? 0 : (size_t)n * sizeof(float);
}

int diffattn_v1_decode(const void* q1, const void* q2, const void* k1_cache, const void* k2_cache,
                       const void* v_cache, const int* cache_len, const float* norm_weight,
                       float* out, void* workspace, size_t workspace_bytes, int B, int S_max,
                       int H, int d, int dv, float lambda, float lambda_init, float eps,
                       diffattn_dtype dtype, void* stream) {
  const char* fn = "diffattn_v1_decode";
  if (!q1 || !q2 || !k1_cache || !k2_cache || !v_cache || !out)
    return fail(DIFFATTN_E_INVALID, "%s: null tensor pointer", fn);
  if (B < 0 || S_max < 0 || H <= 0 || d <= 0 || dv <= 0)
    return fail(DIFFATTN_E_INVALID, "%s: bad sizes B=%d S_max=%d H=%d d=%d dv=%d", fn, B, S_max, H,
                d, dv);
  if (!isfinite(lambda) || !isfinite(lambda_init) || !isfinite(eps) || eps < 0.f)
    return fail(DIFFATTN_E_INVALID, "%s: lambda, lambda_init must be finite and eps finite >= 0", fn);
  if (dtype != DIFFATTN_BF16)
    return fail(dtype == DIFFATTN_F32 ? DIFFATTN_E_UNSUPPORTED : DIFFATTN_E_INVALID,
                "%s: only bf16 is supported", fn);
  if (!((d == 128 && dv == 256) || (d == 64 && dv == 128)))
    return fail(DIFFATTN_E_UNSUPPORTED, "%s: (d=%d, dv=%d) not (128, 256) or (64, 128)", fn, d, dv);
  if (prod({B, S_max, H, dv}) < 0 || prod({B, S_max, H, dv}) > (1LL << 40))
    return fail(DIFFATTN_E_INVALID, "%s: problem too large", fn);
  const void* ptrs[] = {q1, q2, k1_cache, k2_cache, v_cache, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(DIFFATTN_E_ALIGN, "%s: tensor pointers must be 16-byte aligned", fn);
  if ((cache_len && !aligned4(cache_len)) || (norm_weight && !aligned4(norm_weight)))
    return fail(DIFFATTN_E_ALIGN, "%s: cache_len and norm_weight must be 4-byte aligned", fn);
  if (B == 0) return ok();
  const size_t need = diffattn_v1_decode_workspace_bytes(B, S_max, H, d, dv);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(DIFFATTN_E_WORKSPACE, "%s: workspace of %zu bytes required (got %zu%s)", fn, need,
                workspace_bytes, workspace ? "" : ", NULL");
  if (!aligned16(workspace)) return fail(DIFFATTN_E_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  diffattn::V1DecodeArgs a{};
  a.q1 = static_cast<const uint16_t*>(q1);
  a.q2 = static_cast<const uint16_t*>(q2);
  a.k1 = static_cast<const uint16_t*>(k1_cache);
  a.k2 = static_cast<const uint16_t*>(k2_cache);
  a.v = static_cast<const uint16_t*>(v_cache);
  a.cache_len = cache_len;
  a.norm_weight = norm_weight;
  a.out = out;
  a.partial = static_cast<float*>(workspace);
  a.B = B;
  a.S_max = S_max;
  a.H = H;
  a.d = d;
  a.dv = dv;
  diffattn::v1_decode_split(B, S_max, H, &a.split_len, &a.nsplit);
  a.lambda = lambda;
  a.lambda_init = lambda_init;
  a.eps = eps;
  a.scale = 1.0f / sqrtf((float)d);
  return from_hip(diffattn::launch_v1_decode(a, static_cast<hipStream_t>(stream)), fn);
}

size_t diffattn_v2_decode_workspace_bytes(int B, int S_max, int Hq, int Hkv, int d) {
  return diffattn_gda_decode_workspace_bytes(B, S_max, Hq, Hkv, d, 1);
}

// The partials hold every query head's (m, l, o) per slice of the cache, so the
// size does not depend on how the heads are grouped into blocks.
size_t diffattn_gda_decode_workspace_bytes(int B, int S_max, int Hq, int Hkv, int d, int ratio) {
  if (B < 0 || S_max < 0 || Hq <= 0 || Hkv <= 0 || ratio < 1 || ratio > 15) return 0;
  if (Hq % Hkv || (Hq / Hkv) % (ratio + 1) || Hq / Hkv > 16) return 0;
  if (d != 64 && d != 128) return 0;
  int split_len, nsplit, nparts;
  diffattn::decode_split(B, S_max, Hkv, &split_len, &nsplit, &nparts);
  const long long n = prod({B, Hq, nparts, d + 4});
  return n < 0 ? 0 : (size_t)n * sizeof(float);
}

}  // extern "C"

namespace {

// Checks of the V2 decode entry points, before any launch; DIFFATTN_OK or a code.
int v2_decode_check(const char* fn, const void* q, const void* k_cache, const void* v_cache,
                    const int* cache_len, const float* lambda_logit, const void* out, int B,
                    int S_max, int Hq, int Hkv, int d, float scale, diffattn_dtype dtype,
                    int ratio = 1) {
  if (!q || !k_cache || !v_cache || !lambda_logit || !out)
    return fail(DIFFATTN_E_INVALID, "%s: null tensor pointer", fn);
  if (B < 0 || S_max < 0 || Hq <= 0 || Hkv <= 0 || d <= 0)
    return fail(DIFFATTN_E_INVALID, "%s: bad sizes B=%d S_max=%d Hq=%d Hkv=%d d=%d", fn, B, S_max,
                Hq, Hkv, d);
  const int rc = v2_heads_check(fn, Hq, Hkv, d, scale, 0, dtype, ratio);
  if (rc != DIFFATTN_OK) return rc;
  if (Hq / Hkv > 16)
    return fail(DIFFATTN_E_UNSUPPORTED, "%s: Hq/Hkv=%d above 16 query heads per KV head", fn,
                Hq / Hkv);
  if (prod({B, S_max, Hkv, d}) > (1LL << 40)) return fail(DIFFATTN_E_INVALID, "%s: problem too large", fn);
  const void* ptrs[] = {q, k_cache, v_cache, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(DIFFATTN_E_ALIGN, "%s: tensor pointers must be 16-byte aligned", fn);
  if (!aligned4(lambda_logit) || (cache_len && !aligned4(cache_len)))
    return fail(DIFFATTN_E_ALIGN, "%s: lambda_logit and cache_len must be 4-byte aligned", fn);
  return DIFFATTN_OK;
}

int v2_decode_launch(const char* fn, const void* q, const void* k_cache, const void* v_cache,
                     const int* cache_len, const float* lambda_logit, void* out, void* partial,
                     int B, int S_max, int Hq, int Hkv, int d, float scale, void* stream,
                     int ratio = 1) {
  diffattn::DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.cache_len = cache_len;
  a.logit = lambda_logit;
  a.out = static_cast<uint16_t*>(out);
  a.partial = static_cast<float*>(partial);
  a.B = B;
  a.S_max = S_max;
  a.Hq = Hq;
  a.ratio = ratio;
  a.nout = Hq / (ratio + 1) * ratio;
  a.Hkv = Hkv;
  a.d = d;
  int nparts;
  diffattn::decode_split(B, S_max, Hkv, &a.split_len, &a.nsplit, &nparts);
  a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
  return from_hip(diffattn::launch_v2_decode(a, static_cast<hipStream_t>(stream)), fn);
}

}  // namespace

extern "C" {

int diffattn_v2_decode(const void* q, const void* k_cache, const void* v_cache,
                       const int* cache_len, const float* lambda_logit, void* out,
                       void* workspace, size_t workspace_bytes, int B, int S_max, int Hq,
                       int Hkv, int d, float scale, diffattn_dtype dtype, void* stream) {
  const char* fn = "diffattn_v2_decode";
  const int rc = v2_decode_check(fn, q, k_cache, v_cache, cache_len, lambda_logit, out, B, S_max,
                                 Hq, Hkv, d, scale, dtype);
  if (rc != DIFFATTN_OK) return rc;
  if (B == 0) return ok();
  const size_t need = diffattn_v2_decode_workspace_bytes(B, S_max, Hq, Hkv, d);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(DIFFATTN_E_WORKSPACE, "%s: workspace of %zu bytes required (got %zu%s)", fn, need,
                workspace_bytes, workspace ? "" : ", NULL");
  if (!aligned16(workspace)) return fail(DIFFATTN_E_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  return v2_decode_launch(fn, q, k_cache, v_cache, cache_len, lambda_logit, out, workspace, B,
                          S_max, Hq, Hkv, d, scale, stream);
}

int diffattn_gda_decode(const void* q, const void* k_cache, const void* v_cache,
                        const int* cache_len, const float* lambda_logit, void* out,
                        void* workspace, size_t workspace_bytes, int B, int S_max, int Hq,
                        int Hkv, int d, int ratio, float scale, diffattn_dtype dtype,
                        void* stream) {
  const char* fn = "diffattn_gda_decode";
  const int rc = v2_decode_check(fn, q, k_cache, v_cache, cache_len, lambda_logit, out, B, S_max,
                                 Hq, Hkv, d, scale, dtype, ratio);
  if (rc != DIFFATTN_OK) return rc;
  if (B == 0) return ok();
  const size_t need = diffattn_gda_decode_workspace_bytes(B, S_max, Hq, Hkv, d, ratio);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(DIFFATTN_E_WORKSPACE, "%s: workspace of %zu bytes required (got %zu%s)", fn, need,
                workspace_bytes, workspace ? "" : ", NULL");
  if (!aligned16(workspace)) return fail(DIFFATTN_E_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  return v2_decode_launch(fn, q, k_cache, v_cache, cache_len, lambda_logit, out, workspace, B,
                          S_max, Hq, Hkv, d, scale, stream, ratio);
}

int diffattn_v2_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                               const int* cache_len, const float* lambda_logit, void* out, int B,
                               int S_max, int Hq, int Hkv, int d, float scale,
                               diffattn_dtype dtype, void* stream) {
  const char* fn = "diffattn_v2_decode_noalloc";
  const int rc = v2_decode_check(fn, q, k_cache, v_cache, cache_len, lambda_logit, out, B, S_max,
                                 Hq, Hkv, d, scale, dtype);
  if (rc != DIFFATTN_OK) return rc;
  if (B == 0) return ok();
  const size_t need = diffattn_v2_decode_workspace_bytes(B, S_max, Hq, Hkv, d);
  const size_t limit = diffattn::decode_noalloc_scratch_bytes();
  static_assert(DIFFATTN_V2_DECODE_NOALLOC_MAX_BYTES == (size_t(32) << 20),
                "the header's limit is the array's size");
  if (need > limit)
    return fail(DIFFATTN_E_UNSUPPORTED,
                "%s: these sizes need %zu bytes of partial results, above the %zu-byte array of "
                "this entry point; use diffattn_v2_decode with a workspace",
                fn, need, limit);
  hipError_t e = hipSuccess;
  void* scratch = diffattn::decode_noalloc_scratch(&e);
  if (scratch == nullptr) return from_hip(e == hipSuccess ? hipErrorInvalidSymbol : e, fn);
  return v2_decode_launch(fn, q, k_cache, v_cache, cache_len, lambda_logit, out, scratch, B,
                          S_max, Hq, Hkv, d, scale, stream);
}

int diffattn_v2_lambda_proj(const void* x, const void* w_lambda, float* logits, long long N,
                            int d_model, int h, diffattn_dtype dtype, void* stream) {
  const char* fn = "diffattn_v2_lambda_proj";
  if (N < 0 || d_model <= 0 || h <= 0)
    return fail(DIFFATTN_E_INVALID, "%s: bad sizes N=%lld d_model=%d h=%d", fn, N, d_model, h);
  if (dtype != DIFFATTN_BF16)
    return fail(dtype == DIFFATTN_F32 ? DIFFATTN_E_UNSUPPORTED : DIFFATTN_E_INVALID,
                "%s: only bf16 is supported", fn);
  if (h % 16 || h > 64)
    return fail(DIFFATTN_E_UNSUPPORTED, "%s: h=%d must be 16, 32, 48 or 64", fn, h);
  if (d_model % 256)
    return fail(DIFFATTN_E_UNSUPPORTED, "%s: d_model=%d must be a multiple of 256", fn, d_model);
  if (prod({N, d_model}) < 0 || prod({N, d_model}) > (1LL << 40))
    return fail(DIFFATTN_E_INVALID, "%s: problem too large", fn);
  if (N == 0) return ok();
  if (!x || !w_lambda || !logits) return fail(DIFFATTN_E_INVALID, "%s: null tensor pointer", fn);
  if (!aligned16(x) || !aligned16(w_lambda) || !aligned4(logits))
    return fail(DIFFATTN_E_ALIGN, "%s: x and w_lambda must be 16-byte, logits 4-byte aligned", fn);
  diffattn::LambdaProjArgs a{static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_lambda),
                             logits, N, d_model, h};
  return from_hip(diffattn::launch_lambda_proj(a, static_cast<hipStream_t>(stream)), fn);
}

int diffattn_out_proj(const void* attn_out, const void* w_o, void* y, long long M, long long K,
                      long long N, diffattn_dtype dtype, void* stream) {
  const char* fn = "diffattn_out_proj";
  if (M < 0 || K <= 0 || N <= 0)
    return fail(DIFFATTN_E_INVALID, "%s: bad sizes M=%lld K=%lld N=%lld", fn, M, K, N);
  if (dtype != DIFFATTN_BF16)
    return fail(dtype == DIFFATTN_F32 ? DIFFATTN_E_UNSUPPORTED : DIFFATTN_E_INVALID,
                "%s: only bf16 is supported", fn);
  if (K % 64) return fail(DIFFATTN_E_UNSUPPORTED, "%s: K=%lld must be a multiple of 64", fn, K);
  if (N % 4) return fail(DIFFATTN_E_UNSUPPORTED, "%s: N=%lld must be a multiple of 4", fn, N);
  if (prod({M, K}) < 0 || prod({M, N}) < 0 || prod({N, K}) < 0 || prod({M, K}) > (1LL << 40) ||
      prod({M, N}) > (1LL << 40) || K * 256 > 0xffffffffLL)
    return fail(DIFFATTN_E_INVALID, "%s: problem too large", fn);
  if (M == 0) return ok();
  if (!attn_out || !w_o || !y) return fail(DIFFATTN_E_INVALID, "%s: null tensor pointer", fn);
  if (!aligned16(attn_out) || !aligned16(w_o) || !aligned16(y))
    return fail(DIFFATTN_E_ALIGN, "%s: tensor pointers must be 16-byte aligned", fn);
  diffattn::GemmArgs a{static_cast<const uint16_t*>(attn_out), static_cast<const uint16_t*>(w_o),
                       static_cast<uint16_t*>(y), M, N, K};
  return from_hip(diffattn::launch_gemm_tn(a, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"
