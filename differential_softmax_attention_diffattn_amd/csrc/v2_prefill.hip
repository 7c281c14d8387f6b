// DIFF V2 GQA prefill on gfx950 (padded and packed/varlen batches).
//
// Computes, per sequence, query row t and head pair p (heads 2p, 2p+1, which
// share their GQA group's K and V):
//     O_j[t]   = softmax_k(q_{t,j} . k_{k,kv(j)} * scale) v_{k,kv(j)}    (causal: k <= t)
//     out[t,p] = O_2p[t] - sigmoid(logit[t,p]) * O_2p+1[t]
// as described in the "Differential Transformer V2" summary (pogovet.com),
// 상세 정리 §1 and §4: one attention over 2h query heads, even/odd split,
// sigmoid-weighted subtraction, no norm afterwards, h*d output columns.
//
// Work decomposition: a workgroup of 4 waves owns a tile of query rows and PW
// consecutive head pairs of one KV head.  Each wave owns one pair and 32 rows,
// i.e. four 16-column blocks (even/odd head x two row halves).  Every K/V tile
// staged in LDS therefore serves all 2*PW query heads of the workgroup.
//
// Per 64-key tile a wave computes S^T = K Q^T on 16x16x32 bf16 MFMA (keys on
// the M side, query columns on N), so each lane ends up holding one query
// column; the softmax row statistics are then per lane, P^T feeds the second
// MFMA directly as its B operand, and O^T = V^T P^T accumulates with the head
// dim on M.  V is written to LDS transposed (Vt[d][key]) by the loader so the
// A operand reads are two 8-byte LDS loads.  K tiles go global->LDS with
// direct-to-LDS loads into an XOR-swizzled layout.  Rescaling of O is lazy:
// the reference maximum only moves when a column's maximum grows by more than
// 2^8, which keeps P <= 256 (exact in the final O / l quotient).
#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace diffattn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kRows = 32;   // query rows per wave
constexpr int kKeys = 64;   // keys per KV tile
constexpr float kRescaleLog2 = 8.0f;

template <int D>
struct Tile {
  static constexpr int kChunks = D / 8;               // 16-byte chunks per K row
  static constexpr int kKBytes = kKeys * D * 2;       // K tile bytes
  static constexpr int kVtStride = kKeys + 4;         // Vt row length in elements (padded)
  static constexpr int kVtBytes = D * kVtStride * 2;  // Vt tile bytes
  static constexpr int kStage = kKBytes + kVtBytes;
  static constexpr int kKInstr = kKBytes / 1024;      // 1 KiB direct loads per K tile
  static constexpr int kKInstrPerWave = kKInstr / kWaves;
  static constexpr int kVKeysPerThread = D / 32;      // V keys staged per thread
};

__device__ __forceinline__ int k_swizzled(int row, int chunk, int nchunks) {
  return row * nchunks * 16 + ((chunk ^ (row & (nchunks - 1))) << 4);
}

template <int D, int PW, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void v2_prefill_kernel(V2Args a) {
  using TL = Tile<D>;
  constexpr int QSUB = kWaves / PW;
  constexpr int QTILE = kRows * QSUB;
  constexpr int NC = D / 32;   // k-chunks of Q K^T
  constexpr int NDB = D / 16;  // 16-row blocks of O^T
  constexpr int NKT = TL::kVKeysPerThread;

  __shared__ __align__(16) uint8_t smem[2 * TL::kStage];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int c16 = lane & 15;

  // ---- block -> (query tile, sequence, pair group); longest tiles first ----
  const int n_hg = a.Hq / (2 * PW);
  const int per_qt = a.nseq * n_hg;
  const int jr = blockIdx.x / per_qt;
  const int rem = blockIdx.x - jr * per_qt;
  const int seq = rem / n_hg;
  const int hg = rem - seq * n_hg;
  const int n_qt_max = (a.max_seqlen + QTILE - 1) / QTILE;
  const int qt = n_qt_max - 1 - jr;
  int tok0, L;
  if (a.cu_seqlens != nullptr) {
    tok0 = a.cu_seqlens[seq];
    L = a.cu_seqlens[seq + 1] - tok0;
  } else {
    tok0 = seq * a.T;
    L = a.T;
  }
  if (qt < 0 || qt * QTILE >= L) return;  // uniform over the block

  const int hpairs = a.Hq / 2;
  const int group = a.Hq / a.Hkv;
  const int p = hg * PW + (wave % PW);
  const int kv = (hg * PW * 2) / group;
  const int q_lo = qt * QTILE + (wave / PW) * kRows;
  const bool wave_active = q_lo < L;

  const int q_end_block = min(qt * QTILE + QTILE, L);
  const int n_kt = CAUSAL ? (q_end_block - 1) / kKeys + 1 : (L + kKeys - 1) / kKeys;
  const int wave_n_kt =
      !wave_active ? 0 : (CAUSAL ? (min(q_lo + kRows, L) - 1) / kKeys + 1 : n_kt);

  // ---- Q^T fragments (B operand), resident for the whole key loop ----
  u32x4 qf[4][NC];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int head = 2 * p + (nb >> 1);
    const int row = q_lo + (nb & 1) * 16 + c16;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (row < L)
        qf[nb][c] = ldg128(a.q + ((size_t)(tok0 + row) * a.Hq + head) * D + c * 32 + g * 8);
      else
        qf[nb][c] = u32x4{0, 0, 0, 0};
    }
  }

  // ---- loaders ----
  auto load_k_tile = [&](int kt, int stage) {
    uint8_t* base = smem + stage * TL::kStage;
#pragma unroll
    for (int j = 0; j < TL::kKInstrPerWave; ++j) {
      const int blk = wave * TL::kKInstrPerWave + j;
      const int off = blk * 1024 + lane * 16;
      const int row = off / (D * 2);
      const int pos = (off % (D * 2)) >> 4;
      const int chunk = pos ^ (row & (TL::kChunks - 1));
      const int key = min(kt * kKeys + row, L - 1);
      const uint16_t* src = a.k + ((size_t)(tok0 + key) * a.Hkv + kv) * D + chunk * 8;
      __builtin_amdgcn_global_load_lds(
          src, (__attribute__((address_space(3))) void*)(base + blk * 1024), 16, 0, 0);
    }
  };
  const int vdc = threadIdx.x % (D / 8);
  const int vkg = threadIdx.x / (D / 8);
  u32x4 vst[NKT];
  auto load_v_tile = [&](int kt) {
#pragma unroll
    for (int k = 0; k < NKT; ++k) {
      const int key = kt * kKeys + vkg * NKT + k;
      if (key < L)
        vst[k] = ldg128(a.v + ((size_t)(tok0 + key) * a.Hkv + kv) * D + vdc * 8);
      else
        vst[k] = u32x4{0, 0, 0, 0};
    }
  };
  auto store_v_tile = [&](int stage) {
    uint16_t* vt = reinterpret_cast<uint16_t*>(smem + stage * TL::kStage + TL::kKBytes);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint16_t* r0 = vt + (vdc * 8 + 2 * j) * TL::kVtStride + vkg * NKT;
      uint16_t* r1 = r0 + TL::kVtStride;
      if constexpr (NKT == 4) {
        *reinterpret_cast<u32x2*>(r0) =
            u32x2{pack_lo16(vst[0][j], vst[1][j]), pack_lo16(vst[2][j], vst[3][j])};
        *reinterpret_cast<u32x2*>(r1) =
            u32x2{pack_hi16(vst[0][j], vst[1][j]), pack_hi16(vst[2][j], vst[3][j])};
      } else {
        *reinterpret_cast<uint32_t*>(r0) = pack_lo16(vst[0][j], vst[1][j]);
        *reinterpret_cast<uint32_t*>(r1) = pack_hi16(vst[0][j], vst[1][j]);
      }
    }
  };

  // ---- prologue: tile 0 ----
  load_k_tile(0, 0);
  load_v_tile(0);
  store_v_tile(0);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): direct-to-LDS loads landed
  __syncthreads();

  f32x4 o[NDB][4];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) o[db][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref[4], l_part[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    m_ref[nb] = -INFINITY;
    l_part[nb] = 0.f;
  }
  const float cs = a.scale * kLog2e;

  for (int kt = 0; kt < n_kt; ++kt) {
    const int stage = kt & 1;
    const bool has_next = kt + 1 < n_kt;
    if (has_next) {
      load_k_tile(kt + 1, stage ^ 1);
      load_v_tile(kt + 1);
    }
    if (kt < wave_n_kt) {
      const uint8_t* kbase = smem + stage * TL::kStage;
      const uint16_t* vt = reinterpret_cast<const uint16_t*>(kbase + TL::kKBytes);
      const int wave_key_end = CAUSAL ? min(q_lo + kRows, L) : L;
      // two 32-key halves per staged tile keep the score registers small
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int k0 = kt * kKeys + cc * 32;
        if (k0 < wave_key_end) {
          // S^T = K Q^T: 2 key blocks x 4 column blocks
          f32x4 sacc[2][4];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) sacc[kb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
              const u32x4 kf = *reinterpret_cast<const u32x4*>(
                  kbase + k_swizzled(cc * 32 + kb * 16 + c16, c * 4 + g, TL::kChunks));
#pragma unroll
              for (int nb = 0; nb < 4; ++nb) sacc[kb][nb] = mfma_bf16(kf, qf[nb][c], sacc[kb][nb]);
            }
          }

          // causal / ragged mask
          const bool need_mask = (k0 + 32 > L) || (CAUSAL && k0 + 31 > q_lo);
          if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int key = k0 + kb * 16 + 4 * g + i;
                  const int row = q_lo + (nb & 1) * 16 + c16;
                  if (key >= L || (CAUSAL && key > row)) sacc[kb][nb][i] = -INFINITY;
                }
          }

          // online softmax, one query column per lane and column block
          float mt[4];
          bool grow = false;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            float x = sacc[0][nb][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i) x = fmaxf(x, sacc[kb][nb][i]);
            mt[nb] = max_across_rows(x) * cs;
            grow |= mt[nb] > m_ref[nb] + kRescaleLog2;
          }
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) pin_agpr(o[db][nb]);
          if (wave_any(grow)) {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
              const float mn = fmaxf(m_ref[nb], mt[nb]);
              const float alpha = (mn == m_ref[nb]) ? 1.f : fast_exp2(m_ref[nb] - mn);
              m_ref[nb] = mn;
              l_part[nb] *= alpha;
#pragma unroll
              for (int db = 0; db < NDB; ++db) {
                // one accumulator at a time: read, scale, write back
                o[db][nb] *= alpha;
                pin_agpr(o[db][nb]);
                __builtin_amdgcn_sched_barrier(0);
              }
            }
          }
          u32x4 pf[4];
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const float mb = (m_ref[nb] == -INFINITY) ? 0.f : m_ref[nb];
            float pv[8];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float e = fast_exp2(fmaf(sacc[kb][nb][i], cs, -mb));
                pv[kb * 4 + i] = e;
                l_part[nb] += e;
              }
            pf[nb] = u32x4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                           pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
          }

          // O^T += V^T P^T
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const uint16_t* vr = vt + (db * 16 + c16) * TL::kVtStride + cc * 32 + g * 4;
            const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 16);
            const u32x4 vf = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) o[db][nb] = mfma_bf16(vf, pf[nb], o[db][nb]);
          }
        }
      }
    }
    // keep the accumulators in AGPRs across the loop back-edge
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) pin_agpr(o[db][nb]);
    if (has_next) store_v_tile(stage ^ 1);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
  }

  if (!wave_active) return;

  // ---- epilogue: normalise, pair subtraction, bf16 store ----
  float inv[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) inv[nb] = 1.0f / sum_across_rows(l_part[nb]);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int row = q_lo + hf * 16 + c16;
    if (row < L) {
      const size_t tok = (size_t)(tok0 + row);
      const float sg = sigmoid_f32(a.logit[tok * hpairs + p]);
      uint16_t* dst = a.out + (tok * hpairs + p) * D + g * 4;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        float r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ev = __fmul_rn(o[db][hf][i], inv[hf]);
          const float od = __fmul_rn(o[db][hf + 2][i], inv[hf + 2]);
          r[i] = fmaf(-sg, od, ev);
        }
        *reinterpret_cast<u32x2*>(dst + db * 16) =
            u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
      }
    }
  }
}

template <int D, int PW>
hipError_t launch_typed(const V2Args& a, hipStream_t stream) {
  constexpr int QTILE = kRows * (kWaves / PW);
  const int n_qt_max = (a.max_seqlen + QTILE - 1) / QTILE;
  const long long blocks = (long long)n_qt_max * a.nseq * (a.Hq / (2 * PW));
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.causal)
    hipLaunchKernelGGL((v2_prefill_kernel<D, PW, true>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((v2_prefill_kernel<D, PW, false>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const V2Args& a, hipStream_t stream) {
  const int pairs_per_group = (a.Hq / a.Hkv) / 2;
  if (pairs_per_group % 4 == 0) return launch_typed<D, 4>(a, stream);
  if (pairs_per_group % 2 == 0) return launch_typed<D, 2>(a, stream);
  return launch_typed<D, 1>(a, stream);
}

}  // namespace

hipError_t launch_v2_prefill(const V2Args& a, hipStream_t stream) {
  if (a.d == 128) return launch_d<128>(a, stream);
  if (a.d == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace diffattn
