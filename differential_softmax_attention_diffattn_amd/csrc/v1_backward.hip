// DIFF V1 backward on gfx950: gradients of sum(dy * y) of the V1 forward
//     z = (softmax(Q1 K1^T / sqrt d) - lambda softmax(Q2 K2^T / sqrt d)) V,
//     y = (1 - lambda_init) * w * z / sqrt(mean(z^2) + eps)
// ("Differential Transformer | ICLR 2025 Oral" blog, section "Differential
// Attention: 빼기의 힘"; the norm and factor from the V1 recap of the
// "Differential Transformer V2" summary, 상세 정리 §1).  The pages print no
// gradient; this is the chain rule through that forward.  Per (row, head),
// with s = 1 - lambda_init, r = sqrt(mean(z^2) + eps) and g = s w dy:
//     dz = g / r - z <g, z> / (dv r^3),   dw += s dy z / r,   dlambda -= <dz, O2>,
//     dO1 = dz,  dO2 = -lambda dz,
// and for each map the softmax-attention backward with P recomputed from the
// forward's log-sum-exp; both maps read the same V, so dP2 = -lambda dP1 and
// dV = (P1 - lambda P2)^T dz are formed once.
//
// Kernels:
//  * v1_bwd_pre_kernel (16 lanes per row): z from the forward's per-map O, dz
//    (stored bf16 as the MFMA operand), D_k = rowsum(dO_k o O_k) from the
//    rounded dz, log2-unit log-sum-exp, per-block partial sums of dlambda and
//    dw; stats stored [B][H][4][T rounded up to 64] so a tile's row values
//    are contiguous.  v1_bwd_reduce_kernel sums the partials in a fixed order.
//  * v1_bwd_dq_kernel: a wave owns 16 query rows of one (batch, head) and both
//    maps, lanes own query columns; K1, K2 and V tiles of 64 keys stream
//    through LDS: S1^T, S2^T, dP^T = V dz^T, dS^T, dQ_k^T += K_k^T dS_k^T.
//  * v1_bwd_dkdv_kernel: a workgroup of 8 waves owns 128 keys of one (batch,
//    head), a wave 16 keys with their K1 and K2 fragments in registers
//    (lanes own key columns) and V in LDS; Q1, Q2 and dz tiles of 32 rows
//    stream through LDS: S1, S2, dP = dz V^T, dS, dV += (P1 - lambda P2)^T dz,
//    dK_k += dS_k^T Q_k.
// MFMA work is 16x16x32 bf16 with fp32 accumulation; P, dS and dz are rounded
// to bf16 as operands.
#include <math.h>

#include "bwd_common.h"
#include "device_common.h"
#include "kernels.h"

namespace diffattn {
namespace {

using bwd::BTile;
using bwd::load_tile;
using bwd::TileLoader;
using bwd::rows_base;
using bwd::rows_offset;
using bwd::trans_base;
using bwd::trans_offset;

constexpr int kKeys = 64;     // keys per staged tile (dq)
constexpr int kRows = 16;     // query rows per wave (dq)
constexpr int kDqWaves = 8;   // dq: 128 query rows per workgroup
constexpr int kPreBlocks = 1024;  // preprocessing workgroups at most (grid-stride beyond)

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

int pad64(int T) { return (T + 63) / 64 * 64; }

// ---------------------------------------------------------------------------
// Preprocessing: 16 lanes per (row, head), grid-stride; per-block partials.
// ---------------------------------------------------------------------------
constexpr int kPreGroups = 16;  // 16-lane groups per 256-thread workgroup
template <int DV>
__global__ __launch_bounds__(256) void v1_bwd_pre_kernel(V1BwdArgs a, int Tp, uint16_t* dz,
                                                         float* stats, float* part) {
  // A 16-lane group owns one (row, head) at a time; lane l16 holds channels
  // l16*E .. l16*E + E-1, so the group reads each fp32 row as one contiguous
  // run and its dot products are row-of-16 DPP sums (four rows per wave are in
  // flight, no cross-lane traffic through LDS).
  constexpr int E = DV / 16;
  static_assert(E % 4 == 0, "channels per lane in 16-byte vectors");
  const int l16 = threadIdx.x & 15;
  const int grp = threadIdx.x >> 4;
  const float s = 1.0f - a.lambda_init;
  float w[E], dw_acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    w[e] = a.norm_weight ? a.norm_weight[l16 * E + e] : 1.0f;
    dw_acc[e] = 0.f;
  }
  float dl_acc = 0.f;
  const long long n_items = (long long)a.B * a.H * Tp;
  for (long long item = (long long)blockIdx.x * kPreGroups + grp; item < n_items;
       item += (long long)gridDim.x * kPreGroups) {
    const int t = (int)(item % Tp);
    const long long bh = item / Tp;
    const int h = (int)(bh % a.H);
    const int b = (int)(bh / a.H);
    float* st = stats + (size_t)bh * 4 * Tp + t;  // [b][h][k][t] at st[k * Tp]
    if (t >= a.T) {  // padding rows: finite zeros (tiles read and mask them)
      if (l16 == 0) st[0] = st[Tp] = st[2 * Tp] = st[3 * Tp] = 0.f;
      continue;
    }
    const size_t r = ((size_t)b * a.T + t) * a.H + h;
    const float lse1 = a.lse[r * 2], lse2 = a.lse[r * 2 + 1];
    float dy[E], o1[E], o2[E], z[E];
    const size_t c0 = r * DV + l16 * E;
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const f32x4 y4 = *reinterpret_cast<const f32x4*>(a.dy + c0 + e);
      const f32x4 p4 = *reinterpret_cast<const f32x4*>(a.o1 + c0 + e);
      const f32x4 q4 = *reinterpret_cast<const f32x4*>(a.o2 + c0 + e);
#pragma unroll
      for (int i = 0; i < 4; ++i) dy[e + i] = y4[i], o1[e + i] = p4[i], o2[e + i] = q4[i];
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      z[e] = fmaf(-a.lambda, o2[e], o1[e]);  // as the forward forms it
      ss = fmaf(z[e], z[e], ss);
    }
    ss = row16_sum(ss);
    const float rr = sqrtf(ss * (1.0f / DV) + a.eps);
    const float ir = 1.0f / rr;
    float g[E], gz = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      g[e] = s * w[e] * dy[e];
      gz = fmaf(g[e], z[e], gz);
    }
    gz = row16_sum(gz);
    const float cz = gz * ir * ir * ir * (1.0f / DV);
    float d1 = 0.f, d2 = 0.f, dl = 0.f;
    uint32_t zb[E / 2];
#pragma unroll
    for (int e = 0; e < E; e += 2) {
      const float dz0 = fmaf(g[e], ir, -z[e] * cz);
      const float dz1 = fmaf(g[e + 1], ir, -z[e + 1] * cz);
      zb[e / 2] = pack_bf16x2(dz0, dz1);
      const float r0 = bf16lo_to_f32(zb[e / 2]), r1 = bf16hi_to_f32(zb[e / 2]);  // as the MFMAs see dz
      d1 = fmaf(r0, o1[e], d1);
      d1 = fmaf(r1, o1[e + 1], d1);
      d2 = fmaf(r0, o2[e], d2);
      d2 = fmaf(r1, o2[e + 1], d2);
      dl = fmaf(-dz0, o2[e], dl);
      dl = fmaf(-dz1, o2[e + 1], dl);
      dw_acc[e] = fmaf(s * dy[e] * z[e], ir, dw_acc[e]);
      dw_acc[e + 1] = fmaf(s * dy[e + 1] * z[e + 1], ir, dw_acc[e + 1]);
    }
    dl_acc += dl;
    d1 = row16_sum(d1);
    d2 = row16_sum(d2);
    uint32_t* dzr = reinterpret_cast<uint32_t*>(dz + r * DV + l16 * E);
#pragma unroll
    for (int e = 0; e < E / 2; e += 4)
      *reinterpret_cast<u32x4*>(dzr + e) = u32x4{zb[e], zb[e + 1], zb[e + 2], zb[e + 3]};
    if (l16 == 0) {
      st[0] = lse1 * kLog2e;
      st[Tp] = lse2 * kLog2e;
      st[2 * Tp] = d1;
      st[3 * Tp] = -a.lambda * d2;
    }
  }
  // block partials: [dlambda, pad x3, dw[DV]], summed over the groups in order
  __shared__ float red[kPreGroups][DV];
  __shared__ float redl[kPreGroups];
#pragma unroll
  for (int e = 0; e < E; ++e) red[grp][l16 * E + e] = dw_acc[e];
  dl_acc = row16_sum(dl_acc);
  if (l16 == 0) redl[grp] = dl_acc;
  __syncthreads();
  float* pb = part + (size_t)blockIdx.x * (DV + 4);
  for (int c = threadIdx.x; c < DV; c += blockDim.x) {
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < kPreGroups; ++k) acc += red[k][c];
    pb[4 + c] = acc;
  }
  if (threadIdx.x == 0) {
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < kPreGroups; ++k) acc += redl[k];
    pb[0] = acc;
  }
}

// Fixed-order sums of the per-block partials into dlambda and dw: a workgroup
// per 64 partial columns (column 0 is dlambda, 4.. are dw), 16 waves each
// summing every 16th partial row, then the 16 wave sums in order.
constexpr int kRedWaves = 16;
template <int DV>
__global__ __launch_bounds__(kRedWaves * kWave) void v1_bwd_reduce_kernel(V1BwdArgs a,
                                                                         const float* part,
                                                                         int nblk) {
  __shared__ float acc_s[kRedWaves][kWave];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = blockIdx.x * kWave + lane;
  float acc = 0.f;
  if (col < DV + 4) {
#pragma unroll 8
    for (int k = wave; k < nblk; k += kRedWaves) acc += part[(size_t)k * (DV + 4) + col];
  }
  acc_s[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kRedWaves; ++w) t += acc_s[w][lane];
  if (col == 0 && a.dlambda != nullptr) a.dlambda[0] = t;
  if (col >= 4 && col < DV + 4 && a.dnorm_weight != nullptr) a.dnorm_weight[col - 4] = t;
}

// ---------------------------------------------------------------------------
// dQ1 and dQ2: a wave owns 16 query rows of one (batch, head).
// ---------------------------------------------------------------------------
template <int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(kDqWaves * kWave, 1) void v1_bwd_dq_kernel(V1BwdArgs a, int Tp,
                                                                       const uint16_t* dz,
                                                                       const float* stats) {
  using TK = BTile<D>;
  using TV = BTile<DV>;
  constexpr int NC = D / 32;
  constexpr int NCV = DV / 32;
  constexpr int NDB = D / 16;
  constexpr int QTILE = kDqWaves * kRows;
  __shared__ __align__(16) uint8_t k1b0[TK::kBytes];
  __shared__ __align__(16) uint8_t k1b1[TK::kBytes];
  __shared__ __align__(16) uint8_t k2b0[TK::kBytes];
  __shared__ __align__(16) uint8_t k2b1[TK::kBytes];
  __shared__ __align__(16) uint8_t vb0[TV::kBytes];
  __shared__ __align__(16) uint8_t vb1[TV::kBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int T = a.T;
  const int BH = a.B * a.H;
  const int n_qt = (T + QTILE - 1) / QTILE;
  // Longest query tiles first.  When the (batch, head) pairs split evenly
  // over the 8 XCDs (workgroups go to XCDs round robin), each XCD works
  // through its pairs one at a time, all query tiles of a pair together, so
  // that the workgroups running together on it stream the same K1, K2 and V
  // tiles and share them in L2; otherwise longest first over all pairs.
  int jr, bh;
  if (BH % 8 == 0) {
    const int local = blockIdx.x / 8;
    jr = local % n_qt;
    bh = blockIdx.x % 8 + 8 * (local / n_qt);
  } else {
    jr = blockIdx.x / BH;
    bh = blockIdx.x - jr * BH;
  }
  const int qt = n_qt - 1 - jr;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int q_lo = qt * QTILE + wave * kRows;
  const bool wave_active = q_lo < T;
  const int q_end_block = min(qt * QTILE + QTILE, T);
  const int n_kt = CAUSAL ? (q_end_block - 1) / kKeys + 1 : (T + kKeys - 1) / kKeys;
  const int wave_key_end = CAUSAL ? min(q_lo + kRows, T) : T;

  const float cs = kLog2e / sqrtf((float)D);
  const int row = q_lo + c16;  // this lane's query column
  const int rowc = min(row, T - 1);
  const size_t rq = ((size_t)b * T + rowc) * a.H + h;
  u32x4 q1f[NC], q2f[NC], dzf[NCV];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    q1f[c] = ldg128(a.q1 + rq * D + c * 32 + g * 8);
    q2f[c] = ldg128(a.q2 + rq * D + c * 32 + g * 8);
  }
#pragma unroll
  for (int c = 0; c < NCV; ++c) dzf[c] = ldg128(dz + rq * DV + c * 32 + g * 8);
  const float* st = stats + (size_t)bh * 4 * Tp + rowc;
  const float l21 = st[0], l22 = st[Tp], dd1 = st[2 * Tp], dd2 = st[3 * Tp];

  const size_t kstr = (size_t)a.H * D, vstr = (size_t)a.H * DV;
  const uint16_t* k1g = a.k1 + ((size_t)b * T * a.H + h) * D;
  const uint16_t* k2g = a.k2 + ((size_t)b * T * a.H + h) * D;
  const uint16_t* vg = a.v + ((size_t)b * T * a.H + h) * DV;
  const TileLoader<D, true> k_ld(kstr, wave, lane);  // K1 and K2: same layout and stride
  const TileLoader<DV, false> v_ld(vstr, wave, lane);
  auto load_k = [&](int kt, uint8_t* l1, uint8_t* l2) {
    const int r0 = kt * kKeys;
    k_ld.load(k1g + (size_t)r0 * kstr, T - r0, l1, wave, lane);
    k_ld.load(k2g + (size_t)r0 * kstr, T - r0, l2, wave, lane);
  };
  auto load_v = [&](int kt, uint8_t* lv) {
    const int r0 = kt * kKeys;
    v_ld.load(vg + (size_t)r0 * vstr, T - r0, lv, wave, lane);
  };

  f32x4 dq1[NDB], dq2[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dq1[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    dq2[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int tr_key = 4 * g + (c16 >> 2);
  const int tr_byte = 8 * (c16 & 3);
  // the V A-read offsets (16-byte chunk 4c + g of rows c16 and 16 + c16): the
  // most numerous reads of a step, so formed once here and kept in registers
  int vo[2][NCV];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int c = 0; c < NCV; ++c) vo[kb][c] = rows_base<DV>(kb * 16 + c16) ^ (g << 4) ^ (c << 6);

  auto pack8 = [](const float (&x)[8]) {
    return u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                 pack_bf16x2(x[6], x[7])};
  };
  // one 32-key step over the staged tiles
  auto step = [&](auto masked, const uint8_t* l1, const uint8_t* l2, const uint8_t* lv, int cc,
                  int k0) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    // the lane's swizzled row bases, made opaque here so that the offsets
    // derived from them (one XOR each) are formed next to their use instead of
    // being kept live across the loop.  K A reads: 32-byte chunk 2c + (g >> 1),
    // byte 16 (g & 1); V A reads: 16-byte chunk 4c + g (the row layout's
    // swizzle class changes with the 16-key block, hence two bases).
    int bk = trans_base<D>(c16, (g & 1) * 16) ^ ((g >> 1) << 5);
    int tk = trans_base<D>(tr_key, tr_byte);
    asm volatile("" : "+v"(bk), "+v"(tk));
    f32x4 s1[2], s2[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s1[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      s2[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      dp[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int rk = (cc * 32 + kb * 16) * TK::kRowBytes;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int off = (bk ^ (c << 6)) + rk;
        s1[kb] = mfma_bf16(*reinterpret_cast<const u32x4*>(l1 + off), q1f[c], s1[kb]);
        s2[kb] = mfma_bf16(*reinterpret_cast<const u32x4*>(l2 + off), q2f[c], s2[kb]);
      }
#pragma unroll
      for (int c = 0; c < NCV; ++c)
        dp[kb] = mfma_bf16(
            *reinterpret_cast<const u32x4*>(lv + vo[kb][c] + cc * 32 * TV::kRowBytes),
            dzf[c], dp[kb]);
    }
    // K1^T and K2^T fragments of the dQ products (transposing reads), kKtRing
    // blocks ahead of their MFMAs; the first ones go out before dS is formed,
    // and the scheduling fences keep each read where it is issued.  Rows
    // tr_key and tr_key + 16 share a swizzle class: the second read is +16 rows.
    auto fetch_kt = [&](const uint8_t* kl, int db) {
      const int off0 = (tk ^ (db << 5)) + cc * 32 * TK::kRowBytes;
      const u32x2 lo = lds_read_tr16(kl + off0);
      const u32x2 hi = lds_read_tr16(kl + off0 + 16 * TK::kRowBytes);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    constexpr int kKtRing = 2;
    u32x4 k1r[kKtRing], k2r[kKtRing];
#pragma unroll
    for (int i = 0; i < kKtRing; ++i) {
      k1r[i] = fetch_kt(l1, i);
      k2r[i] = fetch_kt(l2, i);
    }
    __builtin_amdgcn_sched_barrier(0);
    float x1[8], x2[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + kb * 16 + 4 * g + i;
        float p1 = fast_exp2(fmaf(s1[kb][i], cs, -l21));
        float p2 = fast_exp2(fmaf(s2[kb][i], cs, -l22));
        if (MASKED) {  // a select, not a branch: every lane takes the same path
          const bool ok = (key < T) & (!CAUSAL | (key <= row));
          p1 = ok ? p1 : 0.f;
          p2 = ok ? p2 : 0.f;
        }
        x1[kb * 4 + i] = p1 * (dp[kb][i] - dd1);
        x2[kb * 4 + i] = p2 * fmaf(-a.lambda, dp[kb][i], -dd2);
      }
    const u32x4 ds1 = pack8(x1), ds2 = pack8(x2);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      dq1[db] = mfma_bf16(k1r[db % kKtRing], ds1, dq1[db]);
      dq2[db] = mfma_bf16(k2r[db % kKtRing], ds2, dq2[db]);
      if (db + kKtRing < NDB) {
        k1r[db % kKtRing] = fetch_kt(l1, db + kKtRing);
        k2r[db % kKtRing] = fetch_kt(l2, db + kKtRing);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // key tiles [0, n_int) are fully valid and visible to every row: unmasked,
  // unrolled by two over fixed LDS objects; the rest take the masked step
  const int n_int = max(0, CAUSAL ? min((qt * QTILE + 1) / kKeys, T / kKeys - 1) : T / kKeys - 1);
  auto interior = [&](int kt, const uint8_t* l1, const uint8_t* l2, const uint8_t* lv, uint8_t* n1,
                      uint8_t* n2, uint8_t* nv) __attribute__((always_inline)) {
    load_k(kt + 1, n1, n2);
    if (wave_active) step(BoolTag<false>{}, l1, l2, lv, 0, kt * kKeys);
    load_v(kt + 1, nv);
    if (wave_active) step(BoolTag<false>{}, l1, l2, lv, 1, kt * kKeys + 32);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
  };
  load_k(0, k1b0, k2b0);
  load_v(0, vb0);
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  int kt = 0;
  for (; kt + 2 <= n_int; kt += 2) {
    interior(kt, k1b0, k2b0, vb0, k1b1, k2b1, vb1);
    interior(kt + 1, k1b1, k2b1, vb1, k1b0, k2b0, vb0);
  }
  if (kt < n_int) {
    interior(kt, k1b0, k2b0, vb0, k1b1, k2b1, vb1);
    ++kt;
  }
  for (; kt < n_kt; ++kt) {
    const bool odd = kt & 1;
    if (kt + 1 < n_kt) {
      if (odd) {
        load_k(kt + 1, k1b0, k2b0);
        load_v(kt + 1, vb0);
      } else {
        load_k(kt + 1, k1b1, k2b1);
        load_v(kt + 1, vb1);
      }
    }
    if (wave_active) {
      const int t0 = kt * kKeys;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        if (t0 + 32 * cc < wave_key_end) {
          if (odd)
            step(BoolTag<true>{}, k1b1, k2b1, vb1, cc, t0 + 32 * cc);
          else
            step(BoolTag<true>{}, k1b0, k2b0, vb0, cc, t0 + 32 * cc);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
  }
  if (!wave_active || row >= T) return;
  const float scale = 1.0f / sqrtf((float)D);
  const size_t ro = (((size_t)b * T + row) * a.H + h) * D + g * 4;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    f32x4 r1, r2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r1[i] = dq1[db][i] * scale;
      r2[i] = dq2[db][i] * scale;
    }
    *reinterpret_cast<f32x4*>(a.dq1 + ro + db * 16) = r1;
    *reinterpret_cast<f32x4*>(a.dq2 + ro + db * 16) = r2;
  }
}

// ---------------------------------------------------------------------------
// dK1, dK2 and dV: a workgroup of 8 waves (two per SIMD, so one wave's MFMAs
// overlap the other's softmax work) owns 128 keys of one (batch, head), a
// wave 16 keys.  Per wave: dK1, dK2 [16 keys x D] and dV [16 keys x DV]
// accumulators and the K1, K2 fragments in registers; V of the 128 keys stays
// in LDS for the whole kernel; Q1, Q2 and dz stream by 32-row tiles.
// ---------------------------------------------------------------------------
constexpr int kKvRows = 32;   // query rows per staged tile (dK/dV)
constexpr int kKvWaves8 = 8;  // waves of the dK/dV workgroup

template <int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(kKvWaves8 * kWave) void v1_bwd_dkdv_kernel(V1BwdArgs a, int Tp,
                                                                       const uint16_t* dz,
                                                                       const float* stats,
                                                                       int cohort) {
  using TK = BTile<D>;
  using TV = BTile<DV>;
  constexpr int NC = D / 32;     // k-steps of the products over d
  constexpr int NCV = DV / 32;   // k-steps over dv
  constexpr int NDB = D / 16;    // 16-column blocks of dK
  constexpr int NDBV = DV / 16;  // 16-column blocks of dV
  constexpr int kKvKeys = kKvWaves8 * 16;
  // per stage: 32-row Q1, Q2 and dz tiles (transposing layout, read both
  // ways), then the rows' log2 lse of both maps and D1, D2 (fp32 x 32 each)
  constexpr int kQB = kKvRows * TK::kRowBytes;
  constexpr int kZB = kKvRows * TV::kRowBytes;
  constexpr int kStage = 2 * kQB + kZB + 4 * kKvRows * 4;
  __shared__ __align__(16) uint8_t vtile[kKvKeys * TV::kRowBytes];
  __shared__ __align__(16) uint8_t st0[kStage];
  __shared__ __align__(16) uint8_t st1[kStage];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int T = a.T;
  const int BH = a.B * a.H;
  const int n_qt = (T + kKvRows - 1) / kKvRows;
  // key tiles with the most query tiles first.  When the (batch, head) pairs
  // split evenly over the 8 XCDs (workgroups go to XCDs round robin), each
  // XCD works through its pairs one at a time, key tiles in order, in rounds
  // of `cohort` workgroups (one per CU): see the item order below.
  int kt, bh, local = -1;
  if (BH % 8 == 0) {
    const int xcd = blockIdx.x % 8;
    local = blockIdx.x / 8;
    const int nkt = (T + kKvKeys - 1) / kKvKeys;
    kt = local % nkt;
    bh = xcd + 8 * (local / nkt);
  } else {
    kt = blockIdx.x / BH;
    bh = blockIdx.x - kt * BH;
  }
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int key0 = kt * kKvKeys;
  const int key_w = key0 + wave * 16;
  const int qt0 = CAUSAL ? key0 / kKvRows : 0;
  // Query tiles.  A round of workgroups that starts together walks them last
  // first (they read the same Q / dz tiles at the same time and share them in
  // L2) and ends one after another; the next round starts one by one, the
  // longest first, each when the others have reached about its first tile,
  // so it walks upwards and stays on their tile.  Only the memory traffic
  // depends on the order.
  const int n_items = n_qt - qt0;
  const bool ascending = local >= 0 && ((local / cohort) & 1);
  auto qt_of = [&](int item) { return ascending ? qt0 + item : n_qt - 1 - item; };

  const int key = key_w + c16;  // this lane's key column
  const int keyc = min(key, T - 1);
  const size_t rk = ((size_t)b * T + keyc) * a.H + h;
  u32x4 k1f[NC], k2f[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    k1f[c] = ldg128(a.k1 + rk * D + c * 32 + g * 8);
    k2f[c] = ldg128(a.k2 + rk * D + c * 32 + g * 8);
  }
  const float cs = kLog2e / sqrtf((float)D);

  const size_t qstr = (size_t)a.H * D, zstr = (size_t)a.H * DV;
  {
    const size_t rv = ((size_t)b * T + key0) * a.H + h;
    load_tile<DV, false, kKvWaves8, kKvKeys>(a.v + rv * DV, zstr, T - key0, vtile, wave, lane);
  }
  // Q1 and Q2 share layout and row stride, so one loader serves both
  const TileLoader<D, true, kKvWaves8, kKvRows> q_ld(qstr, wave, lane);
  const TileLoader<DV, true, kKvWaves8, kKvRows> z_ld(zstr, wave, lane);
  auto load = [&](int item, uint8_t* st) {
    const int r0 = qt_of(item) * kKvRows;
    const size_t rr = ((size_t)b * T + r0) * a.H + h;
    q_ld.load(a.q1 + rr * D, T - r0, st, wave, lane);
    q_ld.load(a.q2 + rr * D, T - r0, st + kQB, wave, lane);
    z_ld.load(dz + rr * DV, T - r0, st + 2 * kQB, wave, lane);
    if (wave < 4 && lane < kKvRows / 4)  // wave k < 4 loads row vector k (128 bytes)
      dma16(stats + ((size_t)bh * 4 + wave) * Tp + r0, (uint32_t)(lane * 16),
            st + 2 * kQB + kZB + wave * kKvRows * 4);
  };

  f32x4 dk1[NDB], dk2[NDB], dvv[NDBV];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk1[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    dk2[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int db = 0; db < NDBV; ++db) dvv[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  // transposing reads (B operands of dV and dK): lane (g, c16) addresses row
  // tr_row (+16 for the second read) and the 4-column chunk tr_byte / 2
  const int tr_row = 4 * g + (c16 >> 2);
  const int tr_byte = 8 * (c16 & 3);
  const int vrow = wave * 16 + c16;

  auto work = [&](int item, const uint8_t* st) __attribute__((always_inline)) {
    const int r0 = qt_of(item) * kKvRows;
    if (CAUSAL && r0 + kKvRows - 1 < key_w) return;  // every key of the wave is above the rows
    const uint8_t* q1l = st;
    const uint8_t* q2l = st + kQB;
    const uint8_t* zl = st + 2 * kQB;
    const float* vec = reinterpret_cast<const float*>(st + 2 * kQB + kZB);
    // the lane's swizzled row bases, made opaque here so that the offsets
    // derived from them (one XOR each) are formed next to their use instead of
    // being kept live across the loop (dozens of registers).  S and dP A reads:
    // 32-byte chunk 2c + (g >> 1), byte 16 (g & 1); V reads: 16-byte chunk 4c + g.
    int bq = trans_base<D>(c16, (g & 1) * 16) ^ ((g >> 1) << 5);
    int bz = trans_base<DV>(c16, (g & 1) * 16) ^ ((g >> 1) << 5);
    int bv = rows_base<DV>(vrow) ^ (g << 4);
    int tz = trans_base<DV>(tr_row, tr_byte);
    int tk = trans_base<D>(tr_row, tr_byte);
    asm volatile("" : "+v"(bq), "+v"(bz), "+v"(bv), "+v"(tz), "+v"(tk));
    float pc[2][4], x1[2][4], x2[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // 16-row blocks of the tile
      f32x4 s1 = f32x4{0.f, 0.f, 0.f, 0.f}, s2 = s1, dp = s1;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int off = (bq ^ (c << 6)) + j * 16 * TK::kRowBytes;
        s1 = mfma_bf16(*reinterpret_cast<const u32x4*>(q1l + off), k1f[c], s1);
        s2 = mfma_bf16(*reinterpret_cast<const u32x4*>(q2l + off), k2f[c], s2);
      }
#pragma unroll
      for (int c = 0; c < NCV; ++c) {
        const u32x4 vb = *reinterpret_cast<const u32x4*>(vtile + (bv ^ (c << 6)));
        dp = mfma_bf16(
            *reinterpret_cast<const u32x4*>(zl + (bz ^ (c << 6)) + j * 16 * TV::kRowBytes), vb, dp);
      }
      const f32x4 l1 = *reinterpret_cast<const f32x4*>(vec + j * 16 + 4 * g);
      const f32x4 l2 = *reinterpret_cast<const f32x4*>(vec + kKvRows + j * 16 + 4 * g);
      const f32x4 e1 = *reinterpret_cast<const f32x4*>(vec + 2 * kKvRows + j * 16 + 4 * g);
      const f32x4 e2 = *reinterpret_cast<const f32x4*>(vec + 3 * kKvRows + j * 16 + 4 * g);
      // result element i: query row r0 + 16 j + 4 g + i, key column c16
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = r0 + j * 16 + 4 * g + i;
        float p1 = fast_exp2(fmaf(s1[i], cs, -l1[i]));
        float p2 = fast_exp2(fmaf(s2[i], cs, -l2[i]));
        // a select, not a branch: every lane takes the same path
        const bool ok = (q < T) & (key < T) & (!CAUSAL | (key <= q));
        p1 = ok ? p1 : 0.f;
        p2 = ok ? p2 : 0.f;
        pc[j][i] = fmaf(-a.lambda, p2, p1);
        x1[j][i] = p1 * (dp[i] - e1[i]);
        x2[j][i] = p2 * fmaf(-a.lambda, dp[i], -e2[i]);
      }
    }
    auto pack = [](const float (&x)[2][4]) {
      return u32x4{pack_bf16x2(x[0][0], x[0][1]), pack_bf16x2(x[0][2], x[0][3]),
                   pack_bf16x2(x[1][0], x[1][1]), pack_bf16x2(x[1][2], x[1][3])};
    };
    // dV += (P1 - lambda P2)^T dz, dK_k += dS_k^T Q_k over the 32 rows; the
    // A operands' eight k slots are rows {4g..4g+3, 16+4g..16+4g+3}, matched by
    // the transposing reads at rows tr_row and tr_row + 16
    const u32x4 pa = pack(pc), sa1 = pack(x1), sa2 = pack(x2);
#pragma unroll
    for (int db = 0; db < NDBV; ++db) {
      // rows tr_row and tr_row + 16 share a swizzle class: the second read is +16 rows
      const int off = tz ^ (db << 5);
      const u32x2 lo = lds_read_tr16(zl + off);
      const u32x2 hi = lds_read_tr16(zl + off + 16 * TV::kRowBytes);
      dvv[db] = mfma_bf16(pa, u32x4{lo[0], lo[1], hi[0], hi[1]}, dvv[db]);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int off0 = tk ^ (db << 5);
      const int off1 = off0 + 16 * TK::kRowBytes;
      const u32x2 a1 = lds_read_tr16(q1l + off0), b1 = lds_read_tr16(q1l + off1);
      const u32x2 a2 = lds_read_tr16(q2l + off0), b2 = lds_read_tr16(q2l + off1);
      dk1[db] = mfma_bf16(sa1, u32x4{a1[0], a1[1], b1[0], b1[1]}, dk1[db]);
      dk2[db] = mfma_bf16(sa2, u32x4{a2[0], a2[1], b2[0], b2[1]}, dk2[db]);
    }
  };

  if (n_items > 0) load(0, st0);
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  int it = 0;
  for (; it + 2 <= n_items; it += 2) {  // unrolled by two: each stage a fixed LDS object
    load(it + 1, st1);
    work(it, st0);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    if (it + 2 < n_items) load(it + 2, st0);
    work(it + 1, st1);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
  }
  if (it < n_items) work(it, st0);

  // result element i: key row key_w + 4 g + i, column 16 db + c16
  const float scale = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kk = key_w + 4 * g + i;
    if (kk >= T) continue;
    const size_t r = ((size_t)b * T + kk) * a.H + h;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      a.dk1[r * D + db * 16 + c16] = dk1[db][i] * scale;
      a.dk2[r * D + db * 16 + c16] = dk2[db][i] * scale;
    }
#pragma unroll
    for (int db = 0; db < NDBV; ++db) a.dvg[r * DV + db * 16 + c16] = dvv[db][i];
  }
}

template <int D, int DV>
struct Layout {
  size_t dz, stats, part;  // byte offsets in the workspace
  size_t total;
  int Tp, nblk;
};

template <int D, int DV>
Layout<D, DV> layout(int B, int T, int H) {
  Layout<D, DV> L;
  L.Tp = pad64(T);
  const long long items = (long long)B * H * L.Tp;
  L.nblk = (int)std::min<long long>(kPreBlocks, (items + kPreGroups - 1) / kPreGroups);
  L.dz = 0;
  L.stats = ((size_t)B * T * H * DV * 2 + 255) / 256 * 256;
  L.part = L.stats + ((size_t)B * H * 4 * L.Tp * 4 + 255) / 256 * 256;
  L.total = L.part + (size_t)L.nblk * (DV + 4) * 4;
  return L;
}

template <int D, int DV>
hipError_t launch_typed(const V1BwdArgs& a, hipStream_t stream) {
  if ((long long)a.B * a.T * a.H == 0) {  // no rows: dlambda and dw are empty sums
    hipLaunchKernelGGL((v1_bwd_reduce_kernel<DV>), dim3((DV + 4 + kWave - 1) / kWave),
                       dim3(kRedWaves * kWave), 0, stream, a, (const float*)nullptr, 0);
    return hipGetLastError();
  }
  const auto L = layout<D, DV>(a.B, a.T, a.H);
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  uint16_t* dz = reinterpret_cast<uint16_t*>(ws + L.dz);
  float* stats = reinterpret_cast<float*>(ws + L.stats);
  float* part = reinterpret_cast<float*>(ws + L.part);
  hipLaunchKernelGGL((v1_bwd_pre_kernel<DV>), dim3(L.nblk), dim3(256), 0, stream, a, L.Tp, dz,
                     stats, part);
  hipLaunchKernelGGL((v1_bwd_reduce_kernel<DV>), dim3((DV + 4 + kWave - 1) / kWave),
                     dim3(kRedWaves * kWave), 0, stream, a, (const float*)part, L.nblk);
  const long long BH = (long long)a.B * a.H;
  const long long dq_blocks = (long long)((a.T + kDqWaves * kRows - 1) / (kDqWaves * kRows)) * BH;
  const long long kv_blocks = (long long)((a.T + kKvWaves8 * 16 - 1) / (kKvWaves8 * 16)) * BH;
  if (dq_blocks > 0x7fffffffLL || kv_blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // dK/dV workgroups that run together on one XCD (one per CU), causal only:
  // without the mask every workgroup has the same work and rounds stay whole
  const int cohort = a.causal ? device_cu_count() / 8 : 0x7fffffff;
  if (a.causal) {
    hipLaunchKernelGGL((v1_bwd_dq_kernel<D, DV, true>), dim3((unsigned)dq_blocks),
                       dim3(kDqWaves * kWave), 0, stream, a, L.Tp, (const uint16_t*)dz,
                       (const float*)stats);
    hipLaunchKernelGGL((v1_bwd_dkdv_kernel<D, DV, true>), dim3((unsigned)kv_blocks),
                       dim3(kKvWaves8 * kWave), 0, stream, a, L.Tp, (const uint16_t*)dz,
                       (const float*)stats, cohort);
  } else {
    hipLaunchKernelGGL((v1_bwd_dq_kernel<D, DV, false>), dim3((unsigned)dq_blocks),
                       dim3(kDqWaves * kWave), 0, stream, a, L.Tp, (const uint16_t*)dz,
                       (const float*)stats);
    hipLaunchKernelGGL((v1_bwd_dkdv_kernel<D, DV, false>), dim3((unsigned)kv_blocks),
                       dim3(kKvWaves8 * kWave), 0, stream, a, L.Tp, (const uint16_t*)dz,
                       (const float*)stats, cohort);
  }
  return hipGetLastError();
}

}  // namespace

size_t v1_bwd_workspace_bytes(int B, int T, int H, int d, int dv) {
  if (d == 128 && dv == 256) return layout<128, 256>(B, T, H).total;
  if (d == 64 && dv == 128) return layout<64, 128>(B, T, H).total;
  return 0;
}

hipError_t launch_v1_backward(const V1BwdArgs& a, hipStream_t stream) {
  if (a.d == 128 && a.dv == 256) return launch_typed<128, 256>(a, stream);
  if (a.d == 64 && a.dv == 128) return launch_typed<64, 128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace diffattn
