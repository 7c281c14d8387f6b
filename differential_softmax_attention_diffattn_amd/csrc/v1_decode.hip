// DIFF V1 decode step on gfx950: one new query row per (batch entry, head)
// against the cached K1, K2 and V:
//     z = softmax_k(q1 . k1_k / sqrt d) V - lambda softmax_k(q2 . k2_k / sqrt d) V,
//     y = (1 - lambda_init) * w * z / sqrt(mean(z^2) + eps),     k < cache_len[b]
// ("Differential Transformer | ICLR 2025 Oral" blog, section "Differential
// Attention: 빼기의 힘"; the norm and factor from the V1 recap of the
// "Differential Transformer V2" summary, 상세 정리 §1).  The step is bound by
// reading the cache: per token and head 2d keys and dv = 2d values.
//
// Split-K.  A workgroup of HW waves owns (batch entry, cache slice, HW heads),
// one head per wave; the waves read adjacent heads of each cached token.  A
// wave walks 32-key chunks: K1 and K2 fragments go straight to registers one
// chunk ahead, the V chunk (32 keys x dv) goes to a per-wave LDS double buffer
// by direct-to-LDS loads and is read back as the V^T MFMA operand with the
// transposing read.  Both maps share the MFMA column block: q1 sits in columns
// 0 and 2 of the first score product and q2 in columns 1 and 3 of the second,
// so lanes of columns 0/2 hold map 1 and 1/3 map 2.  For the P.V product,
// columns 0/1 carry P rounded to bf16 and columns 2/3 the bf16 remainder
// P - bf16(P), so one pass over V gives both maps' outputs with P kept to about
// 16 significant bits (the norm divides by |z|, which is small when the two
// maps nearly cancel, so P needs more than bf16's 8 bits).  Each wave leaves a
// partial (O, m, l) per map; a second kernel merges the partials with
// log-sum-exp weights, forms z and applies the norm and factor.
#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace diffattn {
namespace {

constexpr int kChunk = 32;  // keys per wave step
constexpr float kRescaleLog2 = 8.0f;

// partial record per (batch, head, map, part): O[0..DV), m at DV, l at DV+1, padded
template <int DV>
constexpr int kV1PartStride = DV + 4;

template <int DV>
struct V1DecTile {
  static constexpr int kRowBytes = DV * 2;
  static constexpr int kBytes = kChunk * kRowBytes;  // one V chunk
  static constexpr int kInstr = kBytes / 1024;
};

// V rows: 32-byte chunk c of row r at 32-byte position c ^ (r mod n32).
template <int DV>
__device__ __forceinline__ int v1dec_v_offset(int row, int byte_in_row) {
  constexpr int n32 = DV / 16;
  const int c32 = byte_in_row >> 5;
  return row * V1DecTile<DV>::kRowBytes + ((c32 ^ (row & (n32 - 1))) << 5) + (byte_in_row & 31);
}

int v1_heads_per_block(int H) {
  if (H % 4 == 0) return 4;
  if (H % 2 == 0) return 2;
  return 1;
}

template <int D, int DV, int HW>
__global__ __launch_bounds__(HW * kWave, 1) void v1_decode_split_kernel(V1DecodeArgs a) {
  using TL = V1DecTile<DV>;
  constexpr int NC = D / 32;
  constexpr int NDB = DV / 16;
  // the two halves of each wave's V double buffer are separate LDS objects (the
  // transposing reads of one then need not wait for loads into the other)
  __shared__ __align__(16) uint8_t vbuf0[HW][TL::kBytes];
  __shared__ __align__(16) uint8_t vbuf1[HW][TL::kBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int c16 = lane & 15;

  const int n_hg = a.H / HW;
  const int split = blockIdx.x % a.nsplit;
  const int rest = blockIdx.x / a.nsplit;
  const int hg = rest % n_hg;
  const int b = rest / n_hg;
  const int h = hg * HW + wave;
  int n = a.S_max;
  if (a.cache_len != nullptr) n = min(max(a.cache_len[b], 0), a.S_max);
  const int s0 = split * a.split_len;
  const int s1 = min(s0 + a.split_len, n);
  const int chunks = s1 > s0 ? (s1 - s0 + kChunk - 1) / kChunk : 0;

  // B operands of the two score products: q1 in columns 0 and 2, q2 in 1 and 3
  const bool col1 = c16 == 0 || c16 == 2;
  const bool col2 = c16 == 1 || c16 == 3;
  const int map = c16 & 1;  // the map this lane's column carries (columns 0..3)
  u32x4 qf1[NC], qf2[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const size_t qo = ((size_t)b * a.H + h) * D + c * 32 + g * 8;
    qf1[c] = col1 ? ldg128(a.q1 + qo) : u32x4{0, 0, 0, 0};
    qf2[c] = col2 ? ldg128(a.q2 + qo) : u32x4{0, 0, 0, 0};
  }

  const size_t krow = (size_t)a.H * D;   // elements between consecutive keys
  const size_t vrow = (size_t)a.H * DV;
  const uint16_t* k1base = a.k1 + ((size_t)b * a.S_max * a.H + h) * D;
  const uint16_t* k2base = a.k2 + ((size_t)b * a.S_max * a.H + h) * D;
  // V offsets are 32-bit byte offsets from the slice start (bounded by one slice)
  const uint16_t* vbase = a.v + (((size_t)b * a.S_max + s0) * a.H + h) * DV;

  // rows past the slice end are clamped (their scores are masked), so every load
  // is issued unconditionally and the wait counts stay exact
  auto load_k = [&](int chunk, u32x4 (&k1f)[2][NC], u32x4 (&k2f)[2][NC]) {
    const int base = s0 + chunk * kChunk;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = min(base + kb * 16 + c16, s1 - 1);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        k1f[kb][c] = ldg128(k1base + (size_t)key * krow + c * 32 + g * 8);
        k2f[kb][c] = ldg128(k2base + (size_t)key * krow + c * 32 + g * 8);
      }
    }
  };
  auto load_v = [&](int chunk, uint8_t* dst) {
    const int base = s0 + chunk * kChunk;
#pragma unroll
    for (int j = 0; j < TL::kInstr; ++j) {
      const int off = j * 1024 + lane * 16;
      const int r = off / TL::kRowBytes;
      const int pos = (off % TL::kRowBytes) >> 4;
      constexpr int n32 = DV / 16;
      const int vc = (((pos >> 1) ^ (r & (n32 - 1))) << 1) | (pos & 1);
      const int key = min(base + r, s1 - 1);  // >= s0: loads are only issued for a non-empty slice
      dma16(vbase, (uint32_t)(((size_t)(key - s0) * vrow + vc * 8) * 2), dst + j * 1024);
    }
  };

  f32x4 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, mb = 0.f, l_part = 0.f;  // per lane column (map)
  const float cs = a.scale * kLog2e;
  const int tr_key = 4 * g + (c16 >> 2);
  const int tr_byte = 8 * (c16 & 3);
  const bool lo_col = c16 == 2 || c16 == 3;  // columns carrying P - bf16(P)
  const bool p_col = c16 < 4;

  auto chunk_step = [&](int ci, const u32x4 (&k1f)[2][NC], const u32x4 (&k2f)[2][NC],
                        u32x4 (&k1n)[2][NC], u32x4 (&k2n)[2][NC], const uint8_t* vb,
                        uint8_t* vnext) {
    load_k(ci + 1, k1n, k2n);
    load_v(ci + 1, vnext);
    const int base = s0 + ci * kChunk;
    f32x4 s1acc[2], s2acc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s1acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      s2acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        s1acc[kb] = mfma_bf16(k1f[kb][c], qf1[c], s1acc[kb]);
        s2acc[kb] = mfma_bf16(k2f[kb][c], qf2[c], s2acc[kb]);
      }
    }
    // this lane's map; keys past the slice end and columns beyond 3 are masked
    float sc[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = map ? s2acc[kb][i] : s1acc[kb][i];
        sc[kb][i] = (p_col && base + kb * 16 + 4 * g + i < s1) ? x : -INFINITY;
      }
    float x = sc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) x = fmaxf(x, sc[kb][i]);
    const float mt = max_across_rows(x) * cs;
    if (wave_any(mt > m_ref + kRescaleLog2)) {
      const float mn = fmaxf(m_ref, mt);
      const float alpha = (mn == m_ref) ? 1.f : fast_exp2(m_ref - mn);
      m_ref = mn;
      mb = (mn == -INFINITY) ? 0.f : mn;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
    }
    float pv[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = fast_exp2(fmaf(sc[kb][i], cs, -mb));
        l_part += e;
        // columns 2/3: the part of P that bf16 rounding drops
        pv[kb * 4 + i] = lo_col ? e - bf16_to_f32(f32_to_bf16(e)) : e;
      }
    const u32x4 pf = u32x4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                           pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const u32x2 lo = lds_read_tr16(vb + v1dec_v_offset<DV>(tr_key, db * 32 + tr_byte));
      const u32x2 hi = lds_read_tr16(vb + v1dec_v_offset<DV>(tr_key + 16, db * 32 + tr_byte));
      o[db] = mfma_bf16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf, o[db]);
    }
    // the buffer read here is refilled by the next step's loads
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  };

  u32x4 k1a[2][NC], k2a[2][NC], k1b[2][NC], k2b[2][NC];
  if (chunks > 0) {
    load_k(0, k1a, k2a);
    load_v(0, vbuf0[wave]);
  }
  for (int ci = 0; ci < chunks; ci += 2) {
    chunk_step(ci, k1a, k2a, k1b, k2b, vbuf0[wave], vbuf1[wave]);
    if (ci + 1 < chunks) chunk_step(ci + 1, k1b, k2b, k1a, k2a, vbuf1[wave], vbuf0[wave]);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the unused last prefetch has landed

  // ---- partial (O unnormalised, m in scaled log2 units, l) per map ----
  // O of map e = column e (bf16 P) + column e + 2 (the remainder)
  const float l_tot = sum_across_rows(l_part);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) o[db][i] += __shfl_xor(o[db][i], 2);
  if (c16 < 2) {
    float* dst = a.partial +
                 ((((size_t)b * a.H + h) * 2 + map) * a.nsplit + split) * kV1PartStride<DV>;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<f32x4*>(dst + db * 16 + 4 * g) = o[db];
    if (g == 0) {
      dst[DV] = m_ref;
      dst[DV + 1] = l_tot;
    }
  }
}

// Merge the partials of both maps with log-sum-exp weights, then
// z = O1 - lambda O2 and y = (1 - lambda_init) w z / sqrt(mean z^2 + eps).
template <int DV>
__global__ __launch_bounds__(DV) void v1_decode_combine_kernel(V1DecodeArgs a) {
  __shared__ float wts[2][512];
  __shared__ float inv_l[2];
  __shared__ float red[DV / kWave];
  const int bh = blockIdx.x;
  const int t = threadIdx.x;
  const float* src[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) src[e] = a.partial + ((size_t)bh * 2 + e) * a.nsplit * kV1PartStride<DV>;
  if (t < 2 * kWave) {
    const int e = t / kWave, ln = t % kWave;
    float M = -INFINITY;
    for (int s = ln; s < a.nsplit; s += kWave) M = fmaxf(M, src[e][s * kV1PartStride<DV> + DV]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float L = 0.f;
    for (int s = ln; s < a.nsplit; s += kWave) {
      const float ms = src[e][s * kV1PartStride<DV> + DV];
      const float w = (ms == -INFINITY) ? 0.f : fast_exp2(ms - M);
      wts[e][s] = w;
      L = fmaf(src[e][s * kV1PartStride<DV> + DV + 1], w, L);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
    if (ln == 0) inv_l[e] = L > 0.f ? 1.0f / L : 0.f;
  }
  __syncthreads();
  float res[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    float O = 0.f;
    for (int s = 0; s < a.nsplit; ++s) O = fmaf(src[e][s * kV1PartStride<DV> + t], wts[e][s], O);
    res[e] = __fmul_rn(O, inv_l[e]);
  }
  const float z = fmaf(-a.lambda, res[1], res[0]);
  float ss = z * z;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  ss = 0.f;
#pragma unroll
  for (int w = 0; w < DV / kWave; ++w) ss += red[w];
  // an entry with no cached position (both maps empty) gives zeros
  const bool empty = inv_l[0] == 0.f && inv_l[1] == 0.f;
  const float r = empty ? 0.f : (1.0f - a.lambda_init) / sqrtf(ss * (1.0f / DV) + a.eps);
  const float w = a.norm_weight ? a.norm_weight[t] : 1.0f;
  a.out[(size_t)bh * DV + t] = z * r * w;
}

template <int D, int DV, int HW>
hipError_t launch_typed(const V1DecodeArgs& a, hipStream_t stream) {
  const long long blocks = (long long)a.B * (a.H / HW) * a.nsplit;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((v1_decode_split_kernel<D, DV, HW>), dim3((unsigned)blocks), dim3(HW * kWave),
                     0, stream, a);
  hipLaunchKernelGGL((v1_decode_combine_kernel<DV>), dim3((unsigned)(a.B * a.H)), dim3(DV), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, int DV>
hipError_t launch_dv(const V1DecodeArgs& a, hipStream_t stream) {
  switch (v1_heads_per_block(a.H)) {
    case 4: return launch_typed<D, DV, 4>(a, stream);
    case 2: return launch_typed<D, DV, 2>(a, stream);
    default: return launch_typed<D, DV, 1>(a, stream);
  }
}

}  // namespace

// Slices of 64..4096 keys, aiming for at least four rounds of workgroups over
// the compute units (a workgroup's 128 KB of LDS keeps it alone on its CU;
// one round of long slices measured slower here: 2.27 vs 2.07 ms on B32
// S32768 H12), at most 512 per entry.
void v1_decode_split(int B, int S_max, int H, int* split_len, int* nsplit) {
  const long long units = (long long)B * (H / v1_heads_per_block(H));
  const long long target = 4LL * device_cu_count();
  int len = 4096;
  while (len > 64 && units * ((S_max + len - 1) / len) < target) len /= 2;
  int ns = S_max > 0 ? (S_max + len - 1) / len : 1;
  while (ns > 512) {
    len *= 2;
    ns = (S_max + len - 1) / len;
  }
  *split_len = len;
  *nsplit = ns;
}

hipError_t launch_v1_decode(const V1DecodeArgs& a, hipStream_t stream) {
  if (a.d == 128 && a.dv == 256) return launch_dv<128, 256>(a, stream);
  if (a.d == 64 && a.dv == 128) return launch_dv<64, 128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace diffattn
