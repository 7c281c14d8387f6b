// DIFF V2 backward on gfx950 (padded and packed/varlen batches): gradients of
// sum(dout * out) of the V2 forward
//     O_j[t]   = softmax_k(q_{t,j} . k_{k,kv(j)} * scale) v_{k,kv(j)}    (causal: k <= t)
//     out[t,p] = O_2p[t] - sigmoid(logit[t,p]) * O_2p+1[t]
// ("Differential Transformer V2" summary (pogovet.com), 상세 정리 §1 and §4).
// The pages print no gradient; this is the chain rule through that forward.
// With s = sigmoid(logit):
//     dO_2p = dout_p,   dO_2p+1 = -s dout_p,   dlogit_p = -s (1 - s) <dout_p, O_2p+1>,
// and per query head j the softmax-attention backward
//     D_j = rowsum(dO_j o O_j),  dP = dO_j V^T,  dS = P o (dP - D_j),
//     dQ_j = scale dS K,  dK += scale dS^T Q_j,  dV += P^T dO_j,
// with P recomputed from the forward's log-sum-exp.  Both heads of a pair
// share dout_p, so dout_p V^T is formed once per pair.
//
// Two kernels:
//  * v2_bwd_dq_kernel: the forward's decomposition (a wave owns one pair and
//    16 query rows, lanes own query columns; K and V tiles stream through LDS):
//    S^T = K Q^T, dP^T = V dout^T, dS^T, dQ^T += K^T dS^T.  It first forms its
//    rows' D_2p, D_2p+1, s, dlogit and the log-sum-exp in log2 units, writes
//    dlogit, and stores per head a log-sum-exp and a D value [head][Np] for
//    the next kernel (the odd head's with s folded in): every sequence's rows
//    start at a multiple of 64, so a 32-row query tile's values are one
//    contiguous 128-byte run;
//  * v2_bwd_dkdv_kernel: a workgroup owns 256 keys of one KV head; a wave
//    keeps its 32 keys' K fragments in registers (lanes own key columns), V
//    of the workgroup's keys sits in LDS, and the wave handles both heads of
//    every pair, so dout V^T and the dV product are formed once per pair; the
//    Q and dout tiles of every pair and query tile stream through LDS.
// MFMA work is bf16 with fp32 accumulation (16x16x32 in dQ, 32x32x16 in
// dK/dV); P and dS are rounded to bf16 for the second product of each pair,
// as in the forward.
#include <math.h>

#include "bwd_common.h"
#include "device_common.h"
#include "kernels.h"
#include "varlen.h"

namespace diffattn {
namespace {

using bwd::BTile;
using bwd::load_tile;
using bwd::TileLoader;
using bwd::rows_base;
using bwd::rows_offset;
using bwd::trans_base;
using bwd::trans_offset;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int kKeys = 64;   // keys per staged tile (dq)
constexpr int kRows = 16;   // query rows per wave (dq)

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

// Lane n of each 16-lane row of x, in every lane of that row (DPP
// row_newbcast; n a constant once the caller's loops are unrolled).  Used as
// the first operand of a VOP2 subtraction the compiler folds the broadcast
// into that instruction.
template <int N>
__device__ __forceinline__ float row_bcast_n(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + N, 0xf, 0xf, true));
}
__device__ __forceinline__ float row_bcast(float x, int n) {
  switch (n) {
    case 0: return row_bcast_n<0>(x);
    case 1: return row_bcast_n<1>(x);
    case 2: return row_bcast_n<2>(x);
    case 3: return row_bcast_n<3>(x);
    case 4: return row_bcast_n<4>(x);
    case 5: return row_bcast_n<5>(x);
    case 6: return row_bcast_n<6>(x);
    case 7: return row_bcast_n<7>(x);
    case 8: return row_bcast_n<8>(x);
    case 9: return row_bcast_n<9>(x);
    case 10: return row_bcast_n<10>(x);
    case 11: return row_bcast_n<11>(x);
    case 12: return row_bcast_n<12>(x);
    case 13: return row_bcast_n<13>(x);
    case 14: return row_bcast_n<14>(x);
    default: return row_bcast_n<15>(x);
  }
}

// One sequence of the batch: its first token, length and first workspace row.
struct SeqView {
  long long tok0;
  int L;
  long long ws0;
};

__host__ __device__ __forceinline__ long long pad64(long long x) { return (x + 63) / 64 * 64; }

// Tile t (of `rows`-row tiles, numbered sequence by sequence, a sequence's
// tiles consecutive) -> its sequence and the tile's index inside it.  Returns
// false for a tile that does not exist.  Padded batches divide; packed ones
// number the tiles by slots (varlen.h) and find the sequence by a search over cu_seqlens.
// A packed sequence's workspace rows start at its 64-row slot: 64 * (
// floor(cu[s] / 64) + s), so they fit in floor(N / 64) * 64 + 64 nseq rows.
// WAVE: the whole wave searches together (every lane active, t uniform).
template <bool WAVE>
__device__ __forceinline__ bool tile_of(const V2BwdArgs& a, long long t, int rows, SeqView& sv,
                                        int& tile) {
  if (a.cu_seqlens == nullptr) {
    const int nt = (a.T + rows - 1) / rows;
    const long long b = t / nt;
    if (b >= a.B) return false;
    tile = (int)(t - b * nt);
    sv.tok0 = b * a.T;
    sv.L = a.T;
    sv.ws0 = b * pad64(a.T);
    return true;
  }
  const int s = WAVE ? slot_sequence_wave(a.cu_seqlens, a.nseq, t, rows)
                     : slot_sequence(a.cu_seqlens, a.nseq, t, rows);
  const int c0 = a.cu_seqlens[s];
  const int len = a.cu_seqlens[s + 1] - c0;
  const long long k = t - slot_start(a.cu_seqlens, s, rows);
  if (k >= (len + rows - 1) / rows) return false;
  tile = (int)k;
  sv.tok0 = c0;
  sv.L = len;
  sv.ws0 = 64 * slot_start(a.cu_seqlens, s, 64);
  return true;
}

// ---------------------------------------------------------------------------
// dQ: a wave owns one pair and 16 query rows; K and V tiles of 64 keys stream
// through LDS (K in the transposing layout: it is read both ways).
// ---------------------------------------------------------------------------
template <int D, int PW, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void v2_bwd_dq_kernel(V2BwdArgs a, float* lse2) {
  using TL = BTile<D>;
  constexpr int QSUB = kWaves / PW;
  constexpr int QTILE = kRows * QSUB;
  constexpr int NC = D / 32;
  constexpr int NDB = D / 16;
  __shared__ __align__(16) uint8_t kbuf0[TL::kBytes];
  __shared__ __align__(16) uint8_t kbuf1[TL::kBytes];
  __shared__ __align__(16) uint8_t vbuf0[TL::kBytes];
  __shared__ __align__(16) uint8_t vbuf1[TL::kBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int c16 = lane & 15;

  const int n_hg = a.Hq / (2 * PW);
  const int hg = blockIdx.x % n_hg;
  SeqView sv;
  int qt;
  if (!tile_of<true>(a, blockIdx.x / n_hg, QTILE, sv, qt)) return;  // uniform over the block
  qt = (sv.L + QTILE - 1) / QTILE - 1 - qt;  // a sequence's longest (last) tile first
  const int T = sv.L;
  const long long Np = a.Np;
  const int hpairs = a.Hq / 2;
  const int group = a.Hq / a.Hkv;
  const int p = hg * PW + (wave % PW);
  const int kv = (hg * PW * 2) / group;
  const int q_lo = qt * QTILE + (wave / PW) * kRows;
  const bool wave_active = q_lo < T;
  const int q_end_block = min(qt * QTILE + QTILE, T);
  const int n_kt = CAUSAL ? (q_end_block - 1) / kKeys + 1 : (T + kKeys - 1) / kKeys;
  const int wave_key_end = CAUSAL ? min(q_lo + kRows, T) : T;

  const float cs = a.scale * kLog2e;
  const int row = q_lo + c16;  // this lane's query column
  const int rowc = min(row, T - 1);
  const size_t tok = (size_t)(sv.tok0 + rowc);
  // B operands: Q^T of both heads and dout^T of the pair
  u32x4 qf[2][NC], of[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      qf[nb][c] = ldg128(a.q + (tok * a.Hq + 2 * p + nb) * D + c * 32 + g * 8);
    of[c] = ldg128(a.dout + (tok * hpairs + p) * D + c * 32 + g * 8);
  }
  // The row's values, formed here from the row's O of both heads (read in
  // dout's fragment layout), lse and logit: D_2p = <dout_p, O_2p>,
  // D_2p+1 = -s <dout_p, O_2p+1> (the odd head's output gradient is -s dout_p),
  // dlogit_p = -s (1 - s) <dout_p, O_2p+1> and lse log2(e), with s the pair's
  // sigmoid.  The four lanes of a row (g) each sum 32 of the D products.
  float l2[2], dl[2], sg;
  {
    u32x4 oh[2][NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        oh[nb][c] = ldg128(a.o_heads + (tok * a.Hq + 2 * p + nb) * D + c * 32 + g * 8);
    const float lg = a.logit[tok * hpairs + p];
    const float le = a.lse[tok * a.Hq + 2 * p];
    const float lo = a.lse[tok * a.Hq + 2 * p + 1];
    float de = 0.f, dod = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t gw = of[c][j], ew = oh[0][c][j], ow = oh[1][c][j];
        de = fmaf(bf16lo_to_f32(gw), bf16lo_to_f32(ew), de);
        de = fmaf(bf16hi_to_f32(gw), bf16hi_to_f32(ew), de);
        dod = fmaf(bf16lo_to_f32(gw), bf16lo_to_f32(ow), dod);
        dod = fmaf(bf16hi_to_f32(gw), bf16hi_to_f32(ow), dod);
      }
    de = sum_across_rows(de);
    dod = sum_across_rows(dod);
    sg = sigmoid_f32(lg);
    l2[0] = le * kLog2e;
    l2[1] = lo * kLog2e;
    dl[0] = de;
    dl[1] = -sg * dod;
    // publish them for the dK/dV kernel, whose 32-row query tiles read every
    // row of this tile below the sequence's 32-row bound (rows past the end:
    // finite zeros, which its masks discard).  The odd head's values carry s:
    // its lse in log2 units minus log2(s), so that the dK/dV kernel's
    // exponential gives s P_o directly (0 when s is 0), and <dout_p, O_2p+1>
    // itself, so that dS_o = s P_o (<dout_p, O_2p+1> - dP) needs no s.
    if (g == 0 && row < (T + 31) / 32 * 32) {
      const bool valid = row < T;
      const size_t w = (size_t)(2 * p) * Np + sv.ws0 + row;
      a.delta[w] = valid ? dl[0] : 0.f;
      a.delta[w + Np] = valid ? dod : 0.f;
      lse2[w] = valid ? l2[0] : 0.f;
      lse2[w + Np] = valid ? l2[1] - log2f(sg) : 0.f;
      if (valid) a.dlogit[tok * hpairs + p] = -sg * (1.f - sg) * dod;
    }
  }

  const size_t kv_stride = (size_t)a.Hkv * D;
  const uint16_t* kbase_g = a.k + ((size_t)sv.tok0 * a.Hkv + kv) * D;
  const uint16_t* vbase_g = a.v + ((size_t)sv.tok0 * a.Hkv + kv) * D;
  const TileLoader<D, true> k_ld(kv_stride, wave, lane);
  const TileLoader<D, false> v_ld(kv_stride, wave, lane);
  auto load_k = [&](int kt, uint8_t* kl) {
    const int r0 = kt * kKeys;
    k_ld.load(kbase_g + (size_t)r0 * kv_stride, T - r0, kl, wave, lane);
  };
  auto load_v = [&](int kt, uint8_t* vl) {
    const int r0 = kt * kKeys;
    v_ld.load(vbase_g + (size_t)r0 * kv_stride, T - r0, vl, wave, lane);
  };

  f32x4 dq[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) dq[db][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // transposing-read offsets of the K^T operand (as the forward's V^T)
  const int tr_key = 4 * g + (c16 >> 2);
  const int tr_byte = 8 * (c16 & 3);

  // one 32-key step over the staged tile; MASKED applies the causal / ragged
  // mask (only diagonal and ragged tiles need it)
  auto step = [&](auto masked, const uint8_t* kl, const uint8_t* vl, int cc, int k0)
                  __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    // the lane's swizzled row bases (see the dK/dV kernel): K A reads at
    // 32-byte chunk 2c + (g >> 1), V A reads at 16-byte chunk 4c + g,
    // transposing K reads at row tr_key
    int bk = trans_base<D>(c16, (g & 1) * 16) ^ ((g >> 1) << 5);
    int bv = rows_base<D>(c16) ^ (g << 4);
    int bt = trans_base<D>(tr_key, tr_byte);
    asm volatile("" : "+v"(bk), "+v"(bv), "+v"(bt));
    f32x4 sacc[2][2], dpa[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      dpa[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) sacc[kb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // rows cc 32 + kb 16 + c16: the same swizzle class as c16 in both layouts (D >= 64)
        const int rk = (cc * 32 + kb * 16) * TL::kRowBytes;
        const u32x4 kf = *reinterpret_cast<const u32x4*>(kl + (bk ^ (c << 6)) + rk);
        const u32x4 vf = *reinterpret_cast<const u32x4*>(vl + (bv ^ (c << 6)) + rk);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) sacc[kb][nb] = mfma_bf16(kf, qf[nb][c], sacc[kb][nb]);
        dpa[kb] = mfma_bf16(vf, of[c], dpa[kb]);
      }
    // K^T fragments of the dQ product (transposing reads), kKtRing blocks ahead
    // of their MFMAs; the first ones go out before dS is formed, and the
    // scheduling fences keep each read where it is issued
    auto fetch_kt = [&](int db) {
      const uint8_t* kp = kl + (bt ^ (db << 5)) + cc * 32 * TL::kRowBytes;
      const u32x2 lo = lds_read_tr16(kp);
      const u32x2 hi = lds_read_tr16(kp + 16 * TL::kRowBytes);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    constexpr int kKtRing = 2;
    u32x4 ktr[kKtRing];
#pragma unroll
    for (int i = 0; i < kKtRing; ++i) ktr[i] = fetch_kt(i);
    __builtin_amdgcn_sched_barrier(0);
    // dS^T per head, packed as the B operand of dQ^T += K^T dS^T
    u32x4 dsf[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float v8[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + kb * 16 + 4 * g + i;
          float pr = fast_exp2(fmaf(sacc[kb][nb][i], cs, -l2[nb]));
          if (MASKED && (key >= T || (CAUSAL && key > row))) pr = 0.f;
          const float dpv = nb ? -sg * dpa[kb][i] : dpa[kb][i];
          v8[kb * 4 + i] = pr * (dpv - dl[nb]);
        }
      dsf[nb] = u32x4{pack_bf16x2(v8[0], v8[1]), pack_bf16x2(v8[2], v8[3]),
                      pack_bf16x2(v8[4], v8[5]), pack_bf16x2(v8[6], v8[7])};
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) dq[db][nb] = mfma_bf16(ktr[db % kKtRing], dsf[nb], dq[db][nb]);
      if (db + kKtRing < NDB) ktr[db % kKtRing] = fetch_kt(db + kKtRing);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Key tiles [0, n_int) are fully valid and visible to every row of the
  // workgroup (and each has a full successor): unmasked steps, unrolled by two
  // so each stage is a fixed LDS object, the next tile's K loads before the
  // first step and its V loads before the second.  The rest take the masked step.
  const int n_int = max(0, CAUSAL ? min((qt * QTILE + 1) / kKeys, T / kKeys - 1) : T / kKeys - 1);
  auto interior_tile = [&](int kt, const uint8_t* kl, const uint8_t* vl, uint8_t* kn,
                           uint8_t* vn) __attribute__((always_inline)) {
    load_k(kt + 1, kn);
    if (wave_active) step(BoolTag<false>{}, kl, vl, 0, kt * kKeys);
    load_v(kt + 1, vn);
    if (wave_active) step(BoolTag<false>{}, kl, vl, 1, kt * kKeys + 32);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
  };
  load_k(0, kbuf0);
  load_v(0, vbuf0);
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  int kt = 0;
  for (; kt + 2 <= n_int; kt += 2) {
    interior_tile(kt, kbuf0, vbuf0, kbuf1, vbuf1);
    interior_tile(kt + 1, kbuf1, vbuf1, kbuf0, vbuf0);
  }
  if (kt < n_int) {
    interior_tile(kt, kbuf0, vbuf0, kbuf1, vbuf1);
    ++kt;
  }
  for (; kt < n_kt; ++kt) {
    const bool odd = kt & 1;
    if (kt + 1 < n_kt) {
      if (odd) {
        load_k(kt + 1, kbuf0);
        load_v(kt + 1, vbuf0);
      } else {
        load_k(kt + 1, kbuf1);
        load_v(kt + 1, vbuf1);
      }
    }
    if (wave_active) {
      const int t0 = kt * kKeys;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        if (t0 + 32 * cc < wave_key_end) {
          if (odd)
            step(BoolTag<true>{}, kbuf1, vbuf1, cc, t0 + 32 * cc);
          else
            step(BoolTag<true>{}, kbuf0, vbuf0, cc, t0 + 32 * cc);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
  }
  if (!wave_active || row >= T) return;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float* dst = a.dq + (((size_t)sv.tok0 + row) * a.Hq + 2 * p + nb) * D + g * 4;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      f32x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = dq[db][nb][i] * a.scale;
      *reinterpret_cast<f32x4*>(dst + db * 16) = r;
    }
  }
}

// ---------------------------------------------------------------------------
// dK and dV: a workgroup owns 256 keys of one KV head, a wave 32 of them and
// both heads of every pair.  Per (pair, query tile of 32 rows):
//   S_e, S_o = Q_{e,o} K^T, dP = dout V^T (shared: dP_o = -s dP),
//   dS_e = P_e o (dP - D_e), dS_o = P_o o (-s dP - D_o),
//   dV += (P_e - s P_o)^T dout,  dK += dS_e^T Q_e + dS_o^T Q_o.
// All products are 32x32x16 MFMAs: each LDS operand read (1 KiB per wave)
// feeds 32 x 32 x 16 multiply-adds, half the LDS bytes per FLOP of the
// 16x16x32 form, whose operand reads (the transposing ones above all) held
// the kernel below half its MFMA rate.  The lanes own key columns (32 keys);
// K stays in registers, V of the workgroup's keys in LDS.
// ---------------------------------------------------------------------------
constexpr int kKvRows = 32;               // query rows per staged tile
constexpr int kDkvKeys = kWaves * 32;     // keys per workgroup

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void v2_bwd_dkdv_kernel(V2BwdArgs a, const float* lse2,
                                                                  int cohort) {
  using TL = BTile<D>;
  constexpr int NK = D / 16;  // k-steps over d
  constexpr int NB = D / 32;  // 32-column blocks of dK and dV
  constexpr int kTile = kKvRows * TL::kRowBytes;
  // per stage: Q of the even and odd head and dout of the pair (transposing
  // layout, read both ways), then the rows' lse2 and delta values of both heads
  constexpr int kVec = 4 * kKvRows * 4;
  constexpr int kStage = 3 * kTile + kVec;
  __shared__ __align__(16) uint8_t vt[kDkvKeys * TL::kRowBytes];
  __shared__ __align__(16) uint8_t st0[kStage];
  __shared__ __align__(16) uint8_t st1[kStage];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5;  // half of the wave: k group of the MFMA operands
  const int c32 = lane & 31;

  // blocks: padded batches take the key tiles with the most query tiles first,
  // then (batch, KV head); packed batches go sequence by sequence.  When the
  // (batch, KV head) pairs split evenly over the 8 XCDs (workgroups go to
  // XCDs round robin), each XCD instead works through its pairs one at a
  // time, key tiles in order, so that the workgroups running together on it
  // read the same Q and dout tiles.
  SeqView sv;
  int kt, kvh;
  int local = -1;  // position in its XCD's sequence of workgroups, when ordered so
  if (a.cu_seqlens == nullptr) {
    const int nbg = a.B * a.Hkv;
    int bg;
    if (nbg % 8 == 0) {
      const int nkt = (a.T + kDkvKeys - 1) / kDkvKeys;
      const int xcd = blockIdx.x % 8;
      local = blockIdx.x / 8;
      kt = local % nkt;
      bg = xcd + 8 * (local / nkt);
    } else {
      kt = blockIdx.x / nbg;
      bg = blockIdx.x - kt * nbg;
    }
    const int b = bg / a.Hkv;
    kvh = bg - b * a.Hkv;
    sv.tok0 = (long long)b * a.T;
    sv.L = a.T;
    sv.ws0 = (long long)b * pad64(a.T);
  } else {
    kvh = blockIdx.x % a.Hkv;
    if (!tile_of<true>(a, blockIdx.x / a.Hkv, kDkvKeys, sv, kt)) return;  // uniform over the block
  }
  const int T = sv.L;
  const long long Np = a.Np;
  const int n_qt = (T + kKvRows - 1) / kKvRows;
  const int group = a.Hq / a.Hkv;
  const int npairs = group / 2;
  const int hpairs = a.Hq / 2;
  const int key0 = kt * kDkvKeys;
  const int qt0 = CAUSAL ? key0 / kKvRows : 0;
  // (pair, query tile) items.  An XCD runs `cohort` workgroups at a time (one
  // per CU), in rounds of its sequence: a round that starts together (key
  // tiles in order, so item counts falling) walks the query tiles last first
  // -- its workgroups read the same Q / dout tiles at the same time and share
  // them in L2 -- and ends one workgroup after another; the next round then
  // starts one by one, the longest first, each when the others have reached
  // about its first query tile, so it walks upwards and stays on their tile,
  // and ends together; and so on.  The order changes nothing but the memory
  // traffic: dK and dV sum over all items.
  const int n_items = npairs * (n_qt - qt0);
  const bool ascending = local >= 0 && ((local / cohort) & 1);
  auto qt_of = [&](int item) { return ascending ? qt0 + item / npairs : n_qt - 1 - item / npairs; };

  // V of the workgroup's keys, once (rows past the end clamped; masked below)
  load_tile<D, true, kWaves, kDkvKeys>(a.v + (((size_t)sv.tok0 + key0) * a.Hkv + kvh) * D,
                                       (size_t)a.Hkv * D, T - key0, vt, wave, lane);
  // this lane's key: K^T B operands (column = key, k group hf: d 16 ks + 8 hf .. + 7)
  const int key = key0 + wave * 32 + c32;
  const int keyc = min(key, T - 1);
  const size_t kvrow = ((size_t)sv.tok0 + keyc) * a.Hkv + kvh;
  u32x4 kf[NK];
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) kf[ks] = ldg128(a.k + kvrow * D + ks * 16 + hf * 8);
  const float cs = a.scale * kLog2e;
  const int wave_key_lo = key0 + wave * 32;

  // The stage loads are issued by waves 4-7 only.  Issued by all eight right
  // after the barrier, the direct-to-LDS loads stalled every wave for 600-1000
  // cycles at issue (the CU's address unit takes them one after another) with
  // the MFMA pipes idle; now waves 0-3 start their score MFMAs at once and the
  // two waves of each SIMD run out of step, one's MFMAs under the other's
  // issue stall and softmax.
  constexpr int kLoadWaves = kWaves / 2;
  const int lw = wave - kLoadWaves;  // loading wave index, valid for waves 4-7
  const TileLoader<D, true, kLoadWaves, kKvRows> q_ld((size_t)a.Hq * D, lw, lane);   // Q_e and Q_o
  const TileLoader<D, true, kLoadWaves, kKvRows> o_ld((size_t)hpairs * D, lw, lane);  // dout
  auto load = [&](int item, uint8_t* st) {
    if (wave < kLoadWaves) return;
    const int pp = item % npairs;
    const int qt = qt_of(item);
    const int r0 = qt * kKvRows;
    const int je = kvh * group + 2 * pp;  // even head of the pair
    const int pair = je / 2;
    const uint16_t* qe = a.q + (((size_t)sv.tok0 + r0) * a.Hq + je) * D;
    q_ld.load(qe, T - r0, st, lw, lane);
    q_ld.load(qe + D, T - r0, st + kTile, lw, lane);
    const uint16_t* dsrc = a.dout + (((size_t)sv.tok0 + r0) * hpairs + pair) * D;
    o_ld.load(dsrc, T - r0, st + 2 * kTile, lw, lane);
    // row vectors (32 floats each, padded rows included): 4 x 128 bytes, the
    // lse2 and delta pairs, one by each of waves 4-7
    if (lane < 8) {
      const float* src = lw < 2 ? lse2 + (size_t)(je + lw) * Np : a.delta + (size_t)(je + lw - 2) * Np;
      dma16(src + sv.ws0 + r0, (uint32_t)(lane * 16), st + 3 * kTile + lw * 128);
    }
  };

  f32x16 dk[NB], dv[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) dk[nb][e] = dv[nb][e] = 0.f;
  // transposing reads (B operands of dV and dK, k = query rows): the lane's
  // 16-lane group g4 reads rows 4 hf + (c16 >> 2) (+ 8) of the 16-column
  // block g4 & 1 of each 32-column block; lane c16 gets that block's column
  // c16 down the four rows
  const int c16 = lane & 15;
  const int tr_row = 4 * hf + (c16 >> 2);
  const int tr_byte = 8 * (c16 & 3);
  const int tr_half = ((lane >> 4) & 1) << 5;
  // the query row whose D_e and g_o this lane reads (see the softmax below)
  const int row_lane = 8 * ((lane >> 2) & 3) + 4 * hf + (lane & 3);

  // MASKED: the item's query tile touches the diagonal or a ragged end
  auto work = [&](auto masked, int item, const uint8_t* st) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    const int qt = qt_of(item);
    const int r0 = qt * kKvRows;
    if (CAUSAL && r0 + kKvRows <= wave_key_lo) return;  // every key of the wave is above the rows
    const uint8_t* qle = st;
    const uint8_t* qlo = st + kTile;
    const uint8_t* dl = st + 2 * kTile;
    const float* vec = reinterpret_cast<const float*>(st + 3 * kTile);
    // the lane's swizzled bases, opaque here so that the offsets derived from
    // them (one XOR each) are formed next to their use: A reads at row c32,
    // 32-byte chunk ks, byte 16 hf; V reads the same in the wave's V rows;
    // transposing reads at row tr_row
    int ba = trans_base<D>(c32, hf * 16);
    int bv = ba + wave * 32 * TL::kRowBytes;
    int bt = trans_base<D>(tr_row, tr_byte) ^ tr_half;
    asm volatile("" : "+v"(ba), "+v"(bv), "+v"(bt));
    // S_e, S_o = Q K^T and dP = dout V^T: 32 queries x the wave's 32 keys
    f32x16 se, so, dp;
#pragma unroll
    for (int e = 0; e < 16; ++e) se[e] = so[e] = dp[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const int off = ba ^ (ks << 5);
      const u32x4 qa = *reinterpret_cast<const u32x4*>(qle + off);
      const u32x4 qb = *reinterpret_cast<const u32x4*>(qlo + off);
      const u32x4 da = *reinterpret_cast<const u32x4*>(dl + off);
      const u32x4 vb = *reinterpret_cast<const u32x4*>(vt + (bv ^ (ks << 5)));
      se = mfma32_bf16(qa, kf[ks], se);
      so = mfma32_bf16(qb, kf[ks], so);
      dp = mfma32_bf16(da, vb, dp);
    }
    // P_e, s P_o, their difference P'' = P_e - s P_o and dS of both heads:
    // dS_e = P_e (dP - D_e), dS_o = P_o (-s dP - D_o) = s P_o (g_o - dP) with
    // D_o = -s g_o, g_o = <dout, O_o> (the row values arrive with s folded in:
    // lse2 of the odd head minus log2 s, and g_o).  Element 4 j + i is query
    // r0 + 8 j + 4 hf + i.
    // D_e and g_o: one 4-byte read each, lane 16 r + n holding row
    // 8 (n >> 2) + 4 (r >> 1) + (n & 3), so that lane n = 4 j + i of each
    // 16-lane row holds the row that element 4 j + i of that row's lanes
    // needs; a row broadcast hands it over inside the subtraction (16-byte
    // reads of every lane's 16 rows took 8 KB of LDS reads per item; the
    // log-sum-exp rows stay 16-byte reads, since their broadcast cannot fold
    // into the fused multiply-add of the exponent and costs a move each).
    const float dle_l = vec[2 * kKvRows + row_lane];
    const float go_l = vec[3 * kKvRows + row_lane];
    float pv[16], dse[16], dso[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rv = 8 * j + 4 * hf;
      const f32x4 l2e = *reinterpret_cast<const f32x4*>(vec + rv);
      const f32x4 l2o = *reinterpret_cast<const f32x4*>(vec + kKvRows + rv);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * j + i;
        float pe = fast_exp2(fmaf(se[e], cs, -l2e[i]));
        float po = fast_exp2(fmaf(so[e], cs, -l2o[i]));  // s P_o
        if (MASKED) {  // a select, not a branch: every lane takes the same path
          const int q = r0 + rv + i;
          const bool ok = (q < T) & (key < T) & (!CAUSAL | (key <= q));
          pe = ok ? pe : 0.f;
          po = ok ? po : 0.f;
        }
        pv[e] = pe - po;
        dse[e] = pe * -(row_bcast(dle_l, e) - dp[e]);  // dP - D_e, broadcast operand first
        dso[e] = po * (row_bcast(go_l, e) - dp[e]);
      }
    }
    // dV += P''^T dout and dK += dS_e^T Q_e + dS_o^T Q_o over two 16-query
    // k-steps.  A operands from the registers above (row = key; k slots 0-3
    // are queries 16 s + 4 hf + 0..3, slots 4-7 queries 16 s + 8 + 4 hf +
    // 0..3), B operands by transposing reads of the same rows.
    auto pack8 = [&](const float (&x)[16], int s) {
      return u32x4{pack_bf16x2(x[8 * s + 0], x[8 * s + 1]), pack_bf16x2(x[8 * s + 2], x[8 * s + 3]),
                   pack_bf16x2(x[8 * s + 4], x[8 * s + 5]), pack_bf16x2(x[8 * s + 6], x[8 * s + 7])};
    };
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const u32x4 pa = pack8(pv, s);
      const u32x4 sae = pack8(dse, s);
      const u32x4 sao = pack8(dso, s);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int off = (bt ^ (nb << 6)) + s * 16 * TL::kRowBytes;
        const u32x2 dlo_ = lds_read_tr16(dl + off);
        const u32x2 dhi_ = lds_read_tr16(dl + off + 8 * TL::kRowBytes);
        const u32x2 elo = lds_read_tr16(qle + off);
        const u32x2 ehi = lds_read_tr16(qle + off + 8 * TL::kRowBytes);
        const u32x2 olo = lds_read_tr16(qlo + off);
        const u32x2 ohi = lds_read_tr16(qlo + off + 8 * TL::kRowBytes);
        dv[nb] = mfma32_bf16(pa, u32x4{dlo_[0], dlo_[1], dhi_[0], dhi_[1]}, dv[nb]);
        dk[nb] = mfma32_bf16(sae, u32x4{elo[0], elo[1], ehi[0], ehi[1]}, dk[nb]);
        dk[nb] = mfma32_bf16(sao, u32x4{olo[0], olo[1], ohi[0], ohi[1]}, dk[nb]);
      }
    }
  };

  if (n_items > 0) load(0, st0);
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  auto item_masked = [&](int item) {
    const int r0 = qt_of(item) * kKvRows;
    return (CAUSAL && r0 < key0 + kDkvKeys) || r0 + kKvRows > T || key0 + kDkvKeys > T;
  };
  // One item with the stage chosen at run time: the next item's loads, the
  // work, the wait.  (Reads from a stage chosen at run time wait for every
  // load in flight; only the few masked items take this path.)
  auto one_dynamic = [&](int it) __attribute__((always_inline)) {
    if (it + 1 < n_items) load(it + 1, ((it + 1) & 1) ? st1 : st0);
    work(BoolTag<true>{}, it, (it & 1) ? st1 : st0);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
  };
  // Masked items (the diagonal query tiles and a ragged last one) lie at the
  // two ends of the item order; the unmasked run between them takes the
  // mask-free work in a loop unrolled by two, each stage a fixed LDS object.
  // Separate loops keep each work instance in one register assignment (one
  // loop choosing between a masked and an unmasked instance per item made
  // the compiler copy the dK/dV accumulators between them at every item).
  int m0 = 0, m1 = n_items;
  if (CAUSAL) {
    while (m0 < n_items && item_masked(m0)) ++m0;
    while (m1 > m0 && item_masked(m1 - 1)) --m1;
  } else {
    m0 = m1 = n_items;  // one instance (two make the register allocator spill)
  }
  const int main_b = min(m1, (m0 + 1) & ~1);  // the unrolled run starts at an even item
  const int main_e = main_b + ((m1 - main_b) & ~1);
  for (int it = 0; it < main_b; ++it) one_dynamic(it);
  for (int it = main_b; it < main_e; it += 2) {
    load(it + 1, st1);
    work(BoolTag<false>{}, it, st0);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    if (it + 2 < n_items) load(it + 2, st0);
    work(BoolTag<false>{}, it + 1, st1);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
  }
  for (int it = main_e; it < n_items; ++it) one_dynamic(it);

  // C layout: lane column = d (32 nb + c32), element 4 j + i = key 8 j + 4 hf + i of the wave's 32
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int kk = key0 + wave * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
      if (kk < T) {
        const size_t o = (((size_t)sv.tok0 + kk) * a.Hkv + kvh) * D + nb * 32 + c32;
        a.dk[o] = dk[nb][e] * a.scale;
        a.dv[o] = dv[nb][e];
      }
    }
}

template <int D>
hipError_t launch_d(const V2BwdArgs& a, hipStream_t stream) {
  const long long Np = a.Np;
  float* lse2 = a.delta + (size_t)a.Hq * Np;
  const int pairs_per_group = (a.Hq / a.Hkv) / 2;
  const int PW = pairs_per_group % 4 == 0 ? 4 : pairs_per_group % 2 == 0 ? 2 : 1;
  const int qtile = kRows * (kWaves / PW);
  // tiles over all sequences: padded B * ceil(T / tile); packed the tile slots
  // of varlen.h (blocks of empty slots exit)
  auto tiles = [&](int rows) -> long long {
    if (a.cu_seqlens == nullptr) return (long long)((a.T + rows - 1) / rows) * a.B;
    return slot_count(a.N, a.nseq, 0, rows);
  };
  const long long dq_blocks = tiles(qtile) * (a.Hq / (2 * PW));
  const long long kv_blocks = tiles(kDkvKeys) * a.Hkv;
  // dK/dV workgroups that start together on one XCD (one per CU; padded
  // batches whose (batch, KV head) pairs split evenly over the 8 XCDs)
  const int cohort = (a.cu_seqlens == nullptr && (a.B * a.Hkv) % 8 == 0 && a.causal)
                         ? device_cu_count() / 8
                         : 0x7fffffff;
  if (dq_blocks > 0x7fffffffLL || kv_blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
#define DQ(PWV, C)                                                                               \
  hipLaunchKernelGGL((v2_bwd_dq_kernel<D, PWV, C>), dim3((unsigned)dq_blocks), dim3(kThreads), 0, \
                     stream, a, lse2)
  if (a.causal) {
    if (PW == 4) DQ(4, true);
    else if (PW == 2) DQ(2, true);
    else DQ(1, true);
    hipLaunchKernelGGL((v2_bwd_dkdv_kernel<D, true>), dim3((unsigned)kv_blocks), dim3(kThreads), 0,
                       stream, a, (const float*)lse2, cohort);
  } else {
    if (PW == 4) DQ(4, false);
    else if (PW == 2) DQ(2, false);
    else DQ(1, false);
    hipLaunchKernelGGL((v2_bwd_dkdv_kernel<D, false>), dim3((unsigned)kv_blocks), dim3(kThreads),
                       0, stream, a, (const float*)lse2, cohort);
  }
#undef DQ
  return hipGetLastError();
}

}  // namespace

long long v2_bwd_rows(int B, int T) { return (long long)B * pad64(T); }

long long v2_bwd_varlen_rows(long long N, int nseq) { return pad64(N) + 64LL * nseq; }

size_t v2_bwd_workspace_bytes_rows(long long Np, int Hq) {
  // delta and lse2 [Hq][Np], fp32
  return (size_t)Hq * Np * 2 * sizeof(float);
}

size_t v2_bwd_workspace_bytes(int B, int T, int Hq) {
  return v2_bwd_workspace_bytes_rows(v2_bwd_rows(B, T), Hq);
}

hipError_t launch_v2_backward(const V2BwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_d<128>(a, stream);
  if (a.d == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace diffattn
