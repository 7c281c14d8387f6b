// DIFF V2 decode step on gfx950: one new query row per sequence against the
// KV cache, for every head pair p:
//     O_j   = softmax_k(q_j . k_{k,kv(j)} * scale) v_{k,kv(j)},  k < cache_len[b]
//     out_p = O_2p - sigmoid(logit_p) * O_2p+1
// The KV heads and cache are those of a standard GQA model, so the step reads
// each cached K/V row once per KV head ("Differential Transformer V2" summary,
// 상세 정리 §2: decoding is memory-bound and V2 does not grow the KV cache).
//
// Split-K: a workgroup owns (batch entry, KV head, slice of the cache).  Its 4
// waves walk the slice in 32-key chunks.  All query heads of the KV group
// (up to 16) ride in one MFMA column block, so every K/V byte is read once:
// S^T = K Q^T on 16x16x32 bf16 MFMA with K fragments loaded straight from
// global memory (16-byte loads), then P^T V via a per-wave LDS transpose of V.
// Each workgroup leaves a partial (O, m, l) per query head; a second kernel
// merges the partials with log-sum-exp weights and applies the pair
// subtraction.
#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace diffattn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kChunk = 32;            // keys per wave iteration
constexpr int kVtStride = kChunk + 8;  // bf16 elements per transposed V row (80 B)
constexpr float kRescaleLog2 = 8.0f;

template <int D>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
  constexpr int NC = D / 32;
  constexpr int NDB = D / 16;
  __shared__ __align__(16) uint16_t vts[kWaves][D * kVtStride];
  __shared__ float mrg_m[kWaves][16];
  __shared__ float mrg_l[kWaves][16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int c16 = lane & 15;

  const int split = blockIdx.x % a.nsplit;
  const int bkv = blockIdx.x / a.nsplit;
  const int kv = bkv % a.Hkv;
  const int b = bkv / a.Hkv;
  const int grp = a.Hq / a.Hkv;
  int n = a.S_max;
  if (a.cache_len != nullptr) n = min(max(a.cache_len[b], 0), a.S_max);
  const int t0 = split * a.split_len;
  const int t1 = min(t0 + a.split_len, n);

  // Q^T fragment: column c16 = query head kv*grp + c16 (zeros beyond the group)
  u32x4 qf[NC];
  const bool col_valid = c16 < grp;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (col_valid)
      qf[c] = ldg128(a.q + ((size_t)b * a.Hq + kv * grp + c16) * D + c * 32 + g * 8);
    else
      qf[c] = u32x4{0, 0, 0, 0};
  }

  const size_t row_stride = (size_t)a.Hkv * D;  // elements between consecutive keys
  const uint16_t* kbase = a.k_cache + ((size_t)b * a.S_max * a.Hkv + kv) * D;
  const uint16_t* vbase = a.v_cache + ((size_t)b * a.S_max * a.Hkv + kv) * D;

  f32x4 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_part = 0.f;
  const float cs = a.scale * kLog2e;
  uint16_t* vt = vts[wave];

  // V staging: lane -> keys 8*(lane/16) .. +7 (for D = 128) of the chunk, d-chunk lane % 16
  const int vdc = lane % (D / 8);
  const int vkg = lane / (D / 8);
  constexpr int VKEYS = kChunk / (kWave / (D / 8));  // keys per lane: 8 (D=128) or 4 (D=64)

  for (int base = t0 + wave * kChunk; base < t1; base += kWaves * kChunk) {
    // K fragments straight from global memory
    u32x4 kf[2][NC];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = base + kb * 16 + c16;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        kf[kb][c] = key < t1 ? ldg128(kbase + (size_t)key * row_stride + c * 32 + g * 8)
                             : u32x4{0, 0, 0, 0};
    }
    u32x4 vs[VKEYS];
#pragma unroll
    for (int k = 0; k < VKEYS; ++k) {
      const int key = base + vkg * VKEYS + k;
      vs[k] = key < t1 ? ldg128(vbase + (size_t)key * row_stride + vdc * 8) : u32x4{0, 0, 0, 0};
    }

    f32x4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) sacc[kb] = mfma_bf16(kf[kb][c], qf[c], sacc[kb]);
    }
    if (base + kChunk > t1) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (base + kb * 16 + 4 * g + i >= t1) sacc[kb][i] = -INFINITY;
    }
    float x = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) x = fmaxf(x, sacc[kb][i]);
    const float mt = max_across_rows(x) * cs;
    if (wave_any(mt > m_ref + kRescaleLog2)) {
      const float mn = fmaxf(m_ref, mt);
      const float alpha = (mn == m_ref) ? 1.f : fast_exp2(m_ref - mn);
      m_ref = mn;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
    }
    const float mb = (m_ref == -INFINITY) ? 0.f : m_ref;
    float pv[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = fast_exp2(fmaf(sacc[kb][i], cs, -mb));
        pv[kb * 4 + i] = e;
        l_part += e;
      }
    const u32x4 pf = u32x4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                           pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};

    // transpose the V chunk into this wave's LDS region: vt[d][key]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint16_t* r0 = vt + (vdc * 8 + 2 * j) * kVtStride + vkg * VKEYS;
      uint16_t* r1 = r0 + kVtStride;
      if constexpr (VKEYS == 8) {
        *reinterpret_cast<u32x4*>(r0) =
            u32x4{pack_lo16(vs[0][j], vs[1][j]), pack_lo16(vs[2][j], vs[3][j]),
                  pack_lo16(vs[4][j], vs[5][j]), pack_lo16(vs[6][j], vs[7][j])};
        *reinterpret_cast<u32x4*>(r1) =
            u32x4{pack_hi16(vs[0][j], vs[1][j]), pack_hi16(vs[2][j], vs[3][j]),
                  pack_hi16(vs[4][j], vs[5][j]), pack_hi16(vs[6][j], vs[7][j])};
      } else {
        *reinterpret_cast<u32x2*>(r0) =
            u32x2{pack_lo16(vs[0][j], vs[1][j]), pack_lo16(vs[2][j], vs[3][j])};
        *reinterpret_cast<u32x2*>(r1) =
            u32x2{pack_hi16(vs[0][j], vs[1][j]), pack_hi16(vs[2][j], vs[3][j])};
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): LDS writes done (vmcnt/expcnt unconstrained)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const uint16_t* vr = vt + (db * 16 + c16) * kVtStride + g * 4;
      const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 16);
      o[db] = mfma_bf16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf, o[db]);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next chunk overwrites vt
  }

  // ---- merge the four waves' partial states through LDS ----
  const float l_tot = sum_across_rows(l_part);
  __syncthreads();  // all waves finished with their V regions: reuse them as fp32 O storage
  float* osh = reinterpret_cast<float*>(&vts[0][0]);  // [wave][col 16][D]
  if (g == 0) {
    mrg_m[wave][c16] = m_ref;
    mrg_l[wave][c16] = l_tot;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) osh[(wave * 16 + c16) * D + db * 16 + 4 * g + i] = o[db][i];
  __syncthreads();

  for (int idx = threadIdx.x; idx < grp * D; idx += kThreads) {
    const int col = idx / D;
    const int d = idx - col * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mrg_m[w][col]);
    float O = 0.f, Lsum = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = mrg_m[w][col];
        const float wt = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
        O = fmaf(osh[(w * 16 + col) * D + d], wt, O);
        Lsum = fmaf(mrg_l[w][col], wt, Lsum);
      }
    }
    float* dst = a.partial + (((size_t)b * a.Hq + kv * grp + col) * a.nsplit + split) * (D + 2);
    dst[d] = O;
    if (d == 0) {
      dst[D] = M;
      dst[D + 1] = Lsum;
    }
  }
}

// Merge split partials with log-sum-exp weights, then out_p = O_2p - sigmoid(logit) O_2p+1.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  const int hp = a.Hq / 2;
  const int p = blockIdx.x % hp;
  const int b = blockIdx.x / hp;
  const int d = threadIdx.x;
  float res[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const float* src = a.partial + (((size_t)b * a.Hq + 2 * p + e) * a.nsplit) * (D + 2);
    float M = -INFINITY;
    for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, src[s * (D + 2) + D]);
    float O = 0.f, L = 0.f;
    if (M != -INFINITY) {
      for (int s = 0; s < a.nsplit; ++s) {
        const float ms = src[s * (D + 2) + D];
        const float wt = (ms == -INFINITY) ? 0.f : fast_exp2(ms - M);
        O = fmaf(src[s * (D + 2) + d], wt, O);
        L = fmaf(src[s * (D + 2) + D + 1], wt, L);
      }
    }
    res[e] = (L > 0.f) ? __fdiv_rn(O, L) : 0.f;
  }
  const float sg = sigmoid_f32(a.logit[(size_t)b * hp + p]);
  a.out[((size_t)b * hp + p) * D + d] = f32_to_bf16(fmaf(-sg, res[1], res[0]));
}

template <int D>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  const long long blocks = (long long)a.B * a.Hkv * a.nsplit;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_split_kernel<D>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)(a.B * (a.Hq / 2))), dim3(D), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

void decode_split(int B, int S_max, int Hkv, int* split_len, int* nsplit) {
  // aim for >= 1024 workgroups (4 per CU on 256 CUs), slices of 256..2048 keys
  int len = 2048;
  const long long units = (long long)B * Hkv;
  while (len > 256 && units * ((S_max + len - 1) / len) < 1024) len /= 2;
  *split_len = len;
  *nsplit = S_max > 0 ? (S_max + len - 1) / len : 1;
}

hipError_t launch_v2_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_typed<128>(a, stream);
  if (a.d == 64) return launch_typed<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace diffattn
