// Host-side launch interface between the C ABI (api.cpp) and the HIP kernels.
// Argument validation happens in api.cpp before any of these is called; the
// launchers only pick a kernel instance and a grid, and enqueue on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace diffattn {

struct V1Args {
  const void* q1;
  const void* k1;
  const void* q2;
  const void* k2;
  const void* v;
  const float* norm_weight;  // [dv] or nullptr
  float* out;                // [B,T,H,dv]
  int B, T, H, d, dv;
  float lambda, lambda_init, eps;
  int causal;
  float* o1;                 // fp32 [B,T,H,dv] normalised O of map 1, or nullptr (training forward)
  float* o2;                 // fp32 [B,T,H,dv] normalised O of map 2
  float* lse;                // fp32 [B,T,H,2] natural-log log-sum-exp of both maps
};

// V1 backward.  Gradients of sum(dy * y) of the V1 forward and its norm.
struct V1BwdArgs {
  const uint16_t* q1;        // bf16 [B,T,H,d]
  const uint16_t* k1;
  const uint16_t* q2;
  const uint16_t* k2;
  const uint16_t* v;         // bf16 [B,T,H,dv]
  const float* norm_weight;  // [dv] or nullptr
  const float* o1;           // fp32 [B,T,H,dv] (training forward)
  const float* o2;
  const float* lse;          // fp32 [B,T,H,2]
  const float* dy;           // fp32 [B,T,H,dv]
  float* dq1;                // fp32 [B,T,H,d]
  float* dk1;
  float* dq2;
  float* dk2;
  float* dvg;                // fp32 [B,T,H,dv] (gradient of v)
  float* dlambda;            // fp32 [1]
  float* dnorm_weight;       // fp32 [dv]
  void* workspace;
  int B, T, H, d, dv;
  float lambda, lambda_init, eps;
  int causal;
};

struct V2Args {
  const uint16_t* q;        // bf16 [tokens, Hq, d]
  const uint16_t* k;        // bf16 [tokens, Hkv, d]
  const uint16_t* v;        // bf16 [tokens, Hkv, d]
  const float* logit;       // fp32 [tokens, Hq/2]
  uint16_t* out;            // bf16 [tokens, Hq/2, d]
  const int* cu_seqlens;    // device [nseq+1] or nullptr (padded: sequence s = tokens s*T .. s*T+T-1)
  int nseq;                 // number of sequences (B when padded)
  int max_seqlen;           // longest sequence (T when padded)
  int T;                    // padded sequence length (unused when cu_seqlens != nullptr)
  long long N;              // packed batches: total tokens cu_seqlens[nseq], or -1 if unknown
  int Hq, Hkv, d;
  float scale;              // softmax scale (> 0)
  int causal;
  uint16_t* o_heads;        // bf16 [tokens, Hq, d] per-head outputs, or nullptr (training forward)
  float* lse;               // fp32 [tokens, Hq] natural-log log-sum-exp, or nullptr
  // Heads subtracted: blocks of `ratio` signal heads and one noise head (V2:
  // ratio 1, pairs); output head s subtracts noise head (s / ratio) *
  // (ratio + 1) + ratio from signal head (s / ratio) * (ratio + 1) + s % ratio.
  int ratio = 1;
  int nout = 0;             // output heads: Hq / (ratio + 1) * ratio
};

// V2 backward (padded batches).  Gradients of sum(dout * out) of the V2 forward.
struct V2BwdArgs {
  const uint16_t* q;        // bf16 [B, T, Hq, d]
  const uint16_t* k;        // bf16 [B, T, Hkv, d]
  const uint16_t* v;        // bf16 [B, T, Hkv, d]
  const float* logit;       // fp32 [B, T, Hq/2]
  const uint16_t* o_heads;  // bf16 [B, T, Hq, d]  (from the training forward)
  const float* lse;         // fp32 [B, T, Hq]     (from the training forward)
  const uint16_t* dout;     // bf16 [B, T, Hq/2, d]
  float* dq;                // fp32 [B, T, Hq, d]
  float* dk;                // fp32 [B, T, Hkv, d]
  float* dv;                // fp32 [B, T, Hkv, d]
  float* dlogit;            // fp32 [B, T, Hq/2]
  float* delta;             // fp32 workspace: per-row values, [head][Np] (see v2_backward.hip)
  int B, T, Hq, Hkv, d;
  float scale;
  int causal;
  // packed (varlen) batches: tensors are [N, ...] and sequence s owns tokens
  // cu_seqlens[s] .. cu_seqlens[s+1]-1; nullptr for padded batches (B x T)
  const int* cu_seqlens;
  int nseq;
  long long N;   // packed tokens (varlen)
  long long Np;  // rows per head in the workspace
};

struct DecodeArgs {
  const uint16_t* q;        // bf16 [B, Hq, d]
  const uint16_t* k_cache;  // bf16 [B, S_max, Hkv, d]
  const uint16_t* v_cache;  // bf16 [B, S_max, Hkv, d]
  const int* cache_len;     // device [B] or nullptr
  const float* logit;       // fp32 [B, Hq/2]
  uint16_t* out;            // bf16 [B, Hq/2, d]
  float* partial;           // fp32 workspace [B, Hq, nparts, d + 4]
  int B, S_max, Hq, Hkv, d;
  int split_len, nsplit;    // cache slices of split_len keys; nparts = partials per head
  float scale;
  int ratio = 1;            // signal heads per noise head (as V2Args)
  int nout = 0;             // output heads
};

// Coefficient logits of V2: logits[n, p] = sum_c x[n, c] w[p, c].
struct LambdaProjArgs {
  const uint16_t* x;  // bf16 [N, d_model]
  const uint16_t* w;  // bf16 [h, d_model]
  float* logits;      // fp32 [N, h]
  long long N;
  int d_model, h;     // d_model % 256 == 0, h in {16, 32, 48, 64}
};

// Output projection: y[m, n] = sum_k a[m, k] w[n, k], bf16 out.
struct GemmArgs {
  const uint16_t* a;  // bf16 [M, K]
  const uint16_t* w;  // bf16 [N, K]
  uint16_t* y;        // bf16 [M, N]
  long long M, N, K;  // K % 64 == 0
};

struct V1DecodeArgs {
  const uint16_t* q1;        // bf16 [B, H, d]
  const uint16_t* q2;        // bf16 [B, H, d]
  const uint16_t* k1;        // bf16 [B, S_max, H, d]
  const uint16_t* k2;        // bf16 [B, S_max, H, d]
  const uint16_t* v;         // bf16 [B, S_max, H, dv]
  const int* cache_len;      // device [B] or nullptr
  const float* norm_weight;  // [dv] or nullptr
  float* out;                // fp32 [B, H, dv]
  float* partial;            // fp32 workspace [B, H, 2 maps, nsplit, dv + 4]
  int B, S_max, H, d, dv;
  int split_len, nsplit;     // cache slices of split_len keys
  float lambda, lambda_init, eps, scale;
};

// Compute units of the current device (queried once per device; 256 without one).
int device_cu_count();

// V1 decode split rule shared by the workspace query and the launcher.
void v1_decode_split(int B, int S_max, int H, int* split_len, int* nsplit);
hipError_t launch_v1_decode(const V1DecodeArgs& a, hipStream_t stream);

// Decode split rule shared by the workspace query and the launcher.
void decode_split(int B, int S_max, int Hkv, int* split_len, int* nsplit, int* nparts);

hipError_t launch_v1_f32(const V1Args& a, hipStream_t stream);
// bf16 V1 needs a workspace for V packed as fp16 tiles (see v1_prefill.hip).
size_t v1_bf16_workspace_bytes(int B, int T, int H, int d, int dv);
hipError_t launch_v1_bf16(const V1Args& a, void* workspace, hipStream_t stream);
// V1 backward workspace: dz (bf16), per-row stats and reduction partials (see v1_backward.hip).
size_t v1_bwd_workspace_bytes(int B, int T, int H, int d, int dv);
hipError_t launch_v1_backward(const V1BwdArgs& a, hipStream_t stream);
hipError_t launch_v2_prefill(const V2Args& a, hipStream_t stream);
// V2 backward workspace: per-row delta, log2 lse and sigmoid (see v2_backward.hip).
size_t v2_bwd_workspace_bytes(int B, int T, int Hq);
// Rows per head of that workspace: B * T rounded up per sequence to 64, or for
// packed batches the bound N + 64 * nseq (each sequence padded to 64 rows).
long long v2_bwd_rows(int B, int T);
long long v2_bwd_varlen_rows(long long N, int nseq);
size_t v2_bwd_workspace_bytes_rows(long long Np, int Hq);
hipError_t launch_v2_backward(const V2BwdArgs& a, hipStream_t stream);
hipError_t launch_v2_decode(const DecodeArgs& a, hipStream_t stream);
// The V2 decode's library-owned partials (for callers that cannot allocate):
// its size, and its device address on the current device (looked up once per
// device; nullptr and the HIP error in *err on failure).
size_t decode_noalloc_scratch_bytes();
void* decode_noalloc_scratch(hipError_t* err);
hipError_t launch_lambda_proj(const LambdaProjArgs& a, hipStream_t stream);
hipError_t launch_gemm_tn(const GemmArgs& a, hipStream_t stream);

}  // namespace diffattn
