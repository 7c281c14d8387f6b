// DIFF V1 prefill, fp32 inputs and fp32 arithmetic throughout (FMA pipe).
//
// Same result as the bf16 kernel -- two softmax maps, their lambda-weighted
// difference applied to V, per-head RMS norm over the value channels, then the
// (1 - lambda_init) factor ("Differential Transformer | ICLR 2025 Oral" blog,
// "Differential Attention: 빼기의 힘"; V2 summary 상세 정리 §1 for the norm and
// factor) -- for fp32 workloads, where the contraction is too small to pay
// for MFMA tiling and fp32 accuracy is wanted end to end.
//
// A workgroup of 256 threads owns 16 query rows of one (batch, head); 16
// threads share a row.  Keys are staged in LDS 32 at a time; each thread keeps
// d/16 query values and dv/16 accumulator channels per stream, and the two
// online softmax streams are updated key by key with exact exponentials.
#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace diffattn {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = 16;
constexpr int kKeyTile = 32;
constexpr int kMaxD = 128;
constexpr int kMaxDV = 256;

__global__ __launch_bounds__(kThreads) void v1_f32_kernel(V1Args a) {
  __shared__ float k1s[kKeyTile][kMaxD];
  __shared__ float k2s[kKeyTile][kMaxD];
  __shared__ float vs[kKeyTile][kMaxDV];

  const int D = a.d, DV = a.dv, T = a.T;
  const int nqb = (T + kRowsPerBlock - 1) / kRowsPerBlock;
  const int qb = nqb - 1 - (int)(blockIdx.x / (a.B * a.H));  // longest rows first
  const int bh = blockIdx.x % (a.B * a.H);
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int r = threadIdx.x >> 4;  // row within block
  const int j = threadIdx.x & 15;  // lane within row
  const int row = qb * kRowsPerBlock + r;
  const bool valid = row < T;
  const size_t tok_base = (size_t)b * T;

  const float* q1 = static_cast<const float*>(a.q1);
  const float* q2 = static_cast<const float*>(a.q2);
  const float* k1 = static_cast<const float*>(a.k1);
  const float* k2 = static_cast<const float*>(a.k2);
  const float* v = static_cast<const float*>(a.v);

  const int nd = D / 16, ndv = DV / 16;  // per-thread slices, strided by 16
  float qa[kMaxD / 16], qb2[kMaxD / 16];
#pragma unroll
  for (int i = 0; i < kMaxD / 16; ++i) {
    if (i >= nd) break;
    const size_t off = ((tok_base + (valid ? row : 0)) * a.H + h) * D + j + 16 * i;
    qa[i] = valid ? q1[off] : 0.f;
    qb2[i] = valid ? q2[off] : 0.f;
  }
  float o1[kMaxDV / 16], o2[kMaxDV / 16];
#pragma unroll
  for (int i = 0; i < kMaxDV / 16; ++i) o1[i] = o2[i] = 0.f;
  float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.f, l2 = 0.f;
  const float scale = 1.0f / sqrtf((float)D);

  const int row_end = min(qb * kRowsPerBlock + kRowsPerBlock, T);
  const int key_end = a.causal ? row_end : T;
  const int my_end = a.causal ? row + 1 : T;
  for (int k0 = 0; k0 < key_end; k0 += kKeyTile) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < kKeyTile * D; idx += kThreads) {
      const int kk = idx / D, dd = idx - kk * D;
      const int key = k0 + kk;
      const size_t off = ((tok_base + min(key, T - 1)) * a.H + h) * D + dd;
      k1s[kk][dd] = key < T ? k1[off] : 0.f;
      k2s[kk][dd] = key < T ? k2[off] : 0.f;
    }
    for (int idx = threadIdx.x; idx < kKeyTile * DV; idx += kThreads) {
      const int kk = idx / DV, dd = idx - kk * DV;
      const int key = k0 + kk;
      vs[kk][dd] = key < T ? v[((tok_base + min(key, T - 1)) * a.H + h) * DV + dd] : 0.f;
    }
    __syncthreads();
    const int kn = min(kKeyTile, key_end - k0);
    for (int kk = 0; kk < kn; ++kk) {
      float s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int i = 0; i < kMaxD / 16; ++i) {
        if (i >= nd) break;
        s1 = fmaf(qa[i], k1s[kk][j + 16 * i], s1);
        s2 = fmaf(qb2[i], k2s[kk][j + 16 * i], s2);
      }
      s1 = sum_within_row16(s1) * scale;
      s2 = sum_within_row16(s2) * scale;
      if (k0 + kk < my_end && valid) {
        const float n1 = fmaxf(m1, s1), n2 = fmaxf(m2, s2);
        const float c1 = expf(m1 - n1), c2 = expf(m2 - n2);
        const float p1 = expf(s1 - n1), p2 = expf(s2 - n2);
        l1 = fmaf(l1, c1, p1);
        l2 = fmaf(l2, c2, p2);
        m1 = n1;
        m2 = n2;
#pragma unroll
        for (int i = 0; i < kMaxDV / 16; ++i) {
          if (i >= ndv) break;
          const float vv = vs[kk][j + 16 * i];
          o1[i] = fmaf(o1[i], c1, p1 * vv);
          o2[i] = fmaf(o2[i], c2, p2 * vv);
        }
      }
    }
  }

  // z = O1/l1 - lambda O2/l2, RMS norm over DV channels, (1 - lambda_init) factor
  const float inv1 = 1.0f / l1, inv2 = 1.0f / l2;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxDV / 16; ++i) {
    if (i >= ndv) break;
    const float z = fmaf(-a.lambda, __fmul_rn(o2[i], inv2), __fmul_rn(o1[i], inv1));
    o1[i] = z;
    ss = fmaf(z, z, ss);
  }
  ss = sum_within_row16(ss);
  const float rs = (1.0f - a.lambda_init) / sqrtf(ss / (float)DV + a.eps);
  if (valid) {
    float* dst = a.out + ((tok_base + row) * a.H + h) * DV;
#pragma unroll
    for (int i = 0; i < kMaxDV / 16; ++i) {
      if (i >= ndv) break;
      const int c = j + 16 * i;
      const float w = a.norm_weight ? a.norm_weight[c] : 1.0f;
      dst[c] = o1[i] * rs * w;
    }
  }
}

}  // namespace

hipError_t launch_v1_f32(const V1Args& a, hipStream_t stream) {
  if (a.d % 16 || a.dv % 16 || a.d > kMaxD || a.dv > kMaxDV) return hipErrorInvalidValue;
  const long long blocks = (long long)((a.T + kRowsPerBlock - 1) / kRowsPerBlock) * a.B * a.H;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(v1_f32_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace diffattn
