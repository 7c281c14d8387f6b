// DIFF V1 fused prefill on gfx950, bf16 inputs.
//
// Per (batch, head) and query row t, with the two query/key halves (Q1,K1) and
// (Q2,K2) and values V whose head dim is twice the query/key dim:
//     z_t = sum_k (softmax_k(q1_t.k1_k/sqrt d) - lambda softmax_k(q2_t.k2_k/sqrt d)) v_k
//     y_t = (1 - lambda_init) * w * z_t / sqrt(mean(z_t^2) + eps)
// ("Differential Transformer | ICLR 2025 Oral" blog, section "Differential
// Attention: 빼기의 힘"; the per-head RMS norm and the lambda_init factor are
// from the V1 recap in the "Differential Transformer V2" summary, 상세 정리 §1).
//
// A workgroup of 8 waves owns 128 query rows of one (batch, head): four row
// groups of 32 rows (two 16-column blocks) times the two streams, so each
// wave runs one online softmax, (Q1, K1) or (Q2, K2), over the staged K1/K2/V
// tiles.  Scores are formed transposed, S^T = K Q^T on 16x16x32 bf16 MFMA, so
// one lane holds one query column per block.  P is rounded to fp16 (11-bit
// significand) and P.V runs on 16x16x32 fp16 MFMA: bf16 P would put the
// RMS-normalised output outside a 2e-2 RMS(V) error budget, because the norm
// divides by |z|, which is small when both maps are near-uniform.  A pre-pass
// converts V bf16->fp16 (exact for normal-range values) into a workspace laid
// out tile by tile as Vt[d][key] with padded rows, exactly the LDS image the
// main kernel needs, so V tiles reach LDS by direct-to-LDS loads with no
// register staging or per-tile conversion.  One V^T fragment read from LDS
// feeds two MFMAs (the wave's two column blocks).  At the end the stream-2
// waves hand O2 / l2 to their stream-1 partners through LDS, which apply the
// subtraction, RMS norm and scale in registers; the output is fp32.
#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace diffattn {
namespace {

constexpr int kRowGroups = 4;                 // 32-row groups per workgroup
constexpr int kWaves = 2 * kRowGroups;          // one wave per (stream, row group)
constexpr int kThreads = kWaves * kWave;
constexpr int kRows = 32;
constexpr int kQTile = kRowGroups * kRows;      // 128 query rows per workgroup
constexpr int kKeys = 64;
constexpr float kRescaleLog2 = 8.0f;  // P <= 2^8, well inside fp16 range
constexpr int kVDepth = 2;            // V^T fragments in flight during P.V

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

template <int D, int DV>
struct Tile {
  static constexpr int kChunks = D / 8;
  static constexpr int kKBytes = kKeys * D * 2;       // one of K1 / K2
  static constexpr int kVtRowBytes = kKeys * 2;       // one fp16 Vt row: 64 keys, 128 B
  static constexpr int kVtBytes = DV * kVtRowBytes;
  static constexpr int kStage = 2 * kKBytes + kVtBytes;
  static constexpr int kKInstrPerWave = kKBytes / 1024 / kRowGroups;  // per wave of a stream
  static constexpr int kVInstr = kVtBytes / 1024;   // 1 KiB direct loads per V tile
};

// Packed V tile layout (one per batch, head and 64-key tile): Vt[d][64 keys] in
// fp16, 128 bytes per row, split into eight 16-byte chunks.  Logical chunk c
// (0..7) holds the eight keys one MFMA lane needs for one 32-key half: with
// half = c / 4 and g = c % 4, keys half*32 + 4g + j then half*32 + 16 + 4g + j
// for j = 0..3, so the V^T operand is a single 16-byte LDS read.  Chunk c of
// row d is stored at position c ^ ((d / 2) mod 8), which spreads the 16 rows
// one read instruction touches over all LDS banks.
__device__ __forceinline__ int vt_chunk_offset(int d, int c) {
  return d * 128 + ((c ^ ((d >> 1) & 7)) << 4);
}

// Pre-pass: V [B,T,H,DV] bf16 -> the packed fp16 tiles above (keys past T are zero).
// Thread (dc, c): the 8 rows d = 8 dc .. 8 dc + 7 and logical chunk c.  The
// eight threads of one dc are adjacent, so each store instruction of a wave
// fills whole 128-byte rows.
template <int D, int DV>
__global__ __launch_bounds__(DV) void v1_pack_v_kernel(V1Args a, uint16_t* vp) {
  const int n_kt = (a.T + kKeys - 1) / kKeys;
  const int kt = blockIdx.x % n_kt;
  const int bh = blockIdx.x / n_kt;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const uint16_t* vsrc = static_cast<const uint16_t*>(a.v);
  const int c = threadIdx.x % 8;
  const int dc = threadIdx.x / 8;
  const int key0 = kt * kKeys + (c >> 2) * 32 + 4 * (c & 3);
  u32x4 hv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int key = key0 + (k & 3) + (k >> 2) * 16;
    u32x4 w = u32x4{0, 0, 0, 0};
    if (key < a.T) w = ldg128(vsrc + (((size_t)b * a.T + key) * a.H + h) * DV + dc * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) hv[k][j] = bf16x2_to_f16x2(w[j]);
  }
  uint8_t* vt = reinterpret_cast<uint8_t*>(vp) + (size_t)blockIdx.x * (DV * 128);
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // rows 8 dc + 2j (low halves) and 8 dc + 2j + 1 (high halves)
    const int d0 = dc * 8 + 2 * j;
    *reinterpret_cast<u32x4*>(vt + vt_chunk_offset(d0, c)) =
        u32x4{pack_lo16(hv[0][j], hv[1][j]), pack_lo16(hv[2][j], hv[3][j]),
              pack_lo16(hv[4][j], hv[5][j]), pack_lo16(hv[6][j], hv[7][j])};
    *reinterpret_cast<u32x4*>(vt + vt_chunk_offset(d0 + 1, c)) =
        u32x4{pack_hi16(hv[0][j], hv[1][j]), pack_hi16(hv[2][j], hv[3][j]),
              pack_hi16(hv[4][j], hv[5][j]), pack_hi16(hv[6][j], hv[7][j])};
  }
}

__device__ __forceinline__ int k_swizzled(int row, int chunk, int nchunks) {
  return row * nchunks * 16 + ((chunk ^ (row & (nchunks - 1))) << 4);
}

template <int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void v1_prefill_kernel(V1Args a, const uint16_t* vp) {
  using TL = Tile<D, DV>;
  constexpr int NC = D / 32;
  constexpr int NDB = DV / 16;
  constexpr int XSTRIDE = DV + 4;  // fp32 row stride of the epilogue exchange (banks)
  // two K/V stages during the key loop; the epilogue reuses the space for the exchange
  constexpr int kSmem = 2 * TL::kStage > kQTile * XSTRIDE * 4 ? 2 * TL::kStage
                                                               : kQTile * XSTRIDE * 4;
  __shared__ __align__(16) uint8_t smem[kSmem];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int stream = wave / kRowGroups;  // 0: (Q1, K1), 1: (Q2, K2)
  const int rg = wave % kRowGroups;
  const int g = lane >> 4;
  const int c16 = lane & 15;

  // Block order: query tiles longest first over all (batch, head) pairs, so the
  // short tiles of the causal triangle fill the tail of the launch.  (Grouping
  // one head's tiles per XCD for L2 reuse measured slower: it breaks this
  // longest-first order inside each XCD.)
  const int BH = a.B * a.H;
  const int n_qt = (a.T + kQTile - 1) / kQTile;
  const int jr = blockIdx.x / BH;
  const int bh = blockIdx.x - jr * BH;
  const int qt = n_qt - 1 - jr;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int T = a.T;
  const size_t tok_base = (size_t)b * T;

  const int q_lo = qt * kQTile + rg * kRows;
  const bool wave_active = q_lo < T;
  const int q_end_block = min(qt * kQTile + kQTile, T);
  const int n_kt_all = (T + kKeys - 1) / kKeys;
  const int n_kt = CAUSAL ? (q_end_block - 1) / kKeys + 1 : n_kt_all;
  const int wave_key_end = CAUSAL ? min(q_lo + kRows, T) : T;

  const uint16_t* qsrc = static_cast<const uint16_t*>(stream == 0 ? a.q1 : a.q2);
  const uint16_t* ksrc = static_cast<const uint16_t*>(stream == 0 ? a.k1 : a.k2);

  // Q^T fragments (B operand) of this wave's stream.  (Q is not pre-scaled by
  // log2(e)/sqrt(d): rounding that product to bf16 perturbs the logits enough to
  // show through the difference of two maps and the RMS norm.)
  const float cs = kLog2e / sqrtf((float)D);
  u32x4 qf[2][NC];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int row = q_lo + nb * 16 + c16;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qf[nb][c] = row < T ? ldg128(qsrc + ((tok_base + row) * a.H + h) * D + c * 32 + g * 8)
                          : u32x4{0, 0, 0, 0};
  }

  // K tile of this wave's stream: the four waves of a stream share its 1 KiB
  // loads, wave rg taking blocks rg, rg + 4, ...  Consecutive blocks of a wave
  // lie kJRows rows apart, a multiple of the swizzle period, so a lane fetches
  // the same chunk of each: one 32-bit lane offset serves every load and the
  // tile and block bases move in scalar registers.  Rows past T are clamped on
  // the ragged last tile only (they are masked).
  constexpr int kJRows = kRowGroups * 1024 / (D * 2);
  static_assert(kJRows % TL::kChunks == 0, "K loads must repeat the swizzle");
  const size_t krow_stride = (size_t)a.H * D;  // elements between consecutive tokens
  auto k_lane_chunk = [&](int blk, int& row, int& chunk) {
    const int off = blk * 1024 + lane * 16;
    row = off / (D * 2);
    chunk = ((off % (D * 2)) >> 4) ^ (row & (TL::kChunks - 1));
  };
  uint32_t k_lane_off;  // bytes, first block of a tile
  {
    int row, chunk;
    k_lane_chunk(rg, row, chunk);
    k_lane_off = (uint32_t)((row * krow_stride + chunk * 8) * 2);
  }
  const uint16_t* k_head = ksrc + (tok_base * a.H + h) * D;
  auto load_k_tile = [&](int kt, int stage) {
    uint8_t* base = smem + stage * TL::kStage + stream * TL::kKBytes;
    const uint16_t* tile = k_head + (size_t)kt * kKeys * krow_stride;
    if ((kt + 1) * kKeys <= T) {
#pragma unroll
      for (int j = 0; j < TL::kKInstrPerWave; ++j)
        dma16(tile + (size_t)j * kJRows * krow_stride, k_lane_off,
              base + (rg + kRowGroups * j) * 1024);
    } else {  // ragged last tile: clamp rows past T (they are masked); offsets
              // relative to the tile's first key stay within 32 bits
      const int last = T - 1 - kt * kKeys;
#pragma unroll
      for (int j = 0; j < TL::kKInstrPerWave; ++j) {
        const int blk = rg + kRowGroups * j;
        int row, chunk;
        k_lane_chunk(blk, row, chunk);
        const size_t e = (size_t)min(row, last) * krow_stride + chunk * 8;
        dma16(tile, (uint32_t)(e * 2), base + blk * 1024);
      }
    }
  };
  // V tiles: direct-to-LDS copies of the pre-packed fp16 blocks, spread over all waves
  const uint8_t* vp_bh = reinterpret_cast<const uint8_t*>(vp) + (size_t)bh * n_kt_all * TL::kVtBytes;
  auto load_v_tile = [&](int kt, int stage) {
    uint8_t* base = smem + stage * TL::kStage + 2 * TL::kKBytes;
    const uint8_t* src = vp_bh + (size_t)kt * TL::kVtBytes;
#pragma unroll
    for (int j = 0; j < (TL::kVInstr + kWaves - 1) / kWaves; ++j) {
      const int blk = wave + j * kWaves;
      if (blk < TL::kVInstr) dma16(src, blk * 1024 + lane * 16, base + blk * 1024);
    }
  };

  // Halves of a full tile's loads, for spreading them through a tile's compute.
  // (All eight waves issuing a whole tile at once stalls each of them for
  // hundreds of cycles at the issue of its direct-to-LDS loads.)
  constexpr int kKHalf = (TL::kKInstrPerWave + 1) / 2;
  constexpr int kVPerWave = (TL::kVInstr + kWaves - 1) / kWaves;
  constexpr int kVHalf = (kVPerWave + 1) / 2;
  auto load_k_half = [&](int kt, int stage, int half) __attribute__((always_inline)) {
    uint8_t* base = smem + stage * TL::kStage + stream * TL::kKBytes;
    const uint16_t* tile = k_head + (size_t)kt * kKeys * krow_stride;
#pragma unroll
    for (int j = half * kKHalf; j < min((half + 1) * kKHalf, TL::kKInstrPerWave); ++j)
      dma16(tile + (size_t)j * kJRows * krow_stride, k_lane_off, base + (rg + kRowGroups * j) * 1024);
  };
  auto load_v_half = [&](int kt, int stage, int half) __attribute__((always_inline)) {
    uint8_t* base = smem + stage * TL::kStage + 2 * TL::kKBytes;
    const uint8_t* src = vp_bh + (size_t)kt * TL::kVtBytes;
#pragma unroll
    for (int j = half * kVHalf; j < min((half + 1) * kVHalf, kVPerWave); ++j) {
      const int blk = wave + j * kWaves;
      if (TL::kVInstr % kWaves == 0 || blk < TL::kVInstr)  // (no branch when the loads split evenly)
        dma16(src, blk * 1024 + lane * 16, base + blk * 1024);
    }
  };

  load_k_tile(0, 0);
  load_v_tile(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();

  f32x4 o[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) o[db][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Softmax state per column block (log2 units): m_ref is the reference
  // maximum, -inf until the first key; mb is m_ref with -inf replaced by 0, the
  // value subtracted before exp2.
  float m_ref[2] = {-INFINITY, -INFINITY}, mb[2] = {0.f, 0.f}, l_part[2] = {0.f, 0.f};

  // P = 2^(S cs - ref) for one column block from its two score accumulators:
  // packed fp16 fragment plus the per-lane sum of the rounded values.
  auto probs = [&](const f32x4 (&sacc)[2][2], int nb, float ref, u32x4& pf, float& st)
                   __attribute__((always_inline)) {
    float pv[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[kb * 4 + i] = fast_exp2(fmaf(sacc[kb][nb][i], cs, -ref));
    pf = u32x4{pack_f16x2(pv[0], pv[1]), pack_f16x2(pv[2], pv[3]), pack_f16x2(pv[4], pv[5]),
               pack_f16x2(pv[6], pv[7])};
    st = sum_f16x8(pf, 0.f);
  };

  // One 32-key step of this wave's stream over the staged tile at `stage_base`;
  // MASKED adds the causal / ragged mask (only diagonal and ragged tiles need it).
  //
  // Lazy rescaling, checked after the fact: P = 2^(s - mb) is computed with the
  // current reference; if some lane's eight values sum past 2^8 (so some P may
  // exceed 2^8) or no reference exists yet, the wave takes the rare path: the
  // column maxima are computed, the reference moves up to them, O and l are
  // rescaled and P is recomputed (now <= 1).  Otherwise every P <= 2^8, well
  // inside the fp16 range of P and the fp32 O / l accumulators.
  auto step = [&](auto masked, const uint8_t* stage_base, int cc, int k0, auto mid)
                  __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    const uint8_t* kbase = stage_base + stream * TL::kKBytes;
    const uint8_t* vbytes = stage_base + 2 * TL::kKBytes;
    // S^T = K Q^T for one 32-key half: 2 key blocks x 2 column blocks.  The
    // wave issues them at raised priority, so the score MFMAs of one wave go
    // ahead of the softmax and P.V work of the other wave on its SIMD.
    __builtin_amdgcn_s_setprio(1);
    f32x4 sacc[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) sacc[kb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(
            kbase + k_swizzled(cc * 32 + kb * 16 + c16, c * 4 + g, TL::kChunks));
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) sacc[kb][nb] = mfma_bf16(kf, qf[nb][c], sacc[kb][nb]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    mid();  // work to issue between the score MFMAs and the softmax
    // the first V^T fragments of the P.V product go out before the softmax
    auto fetch_v = [&](int db) {
      return *reinterpret_cast<const u32x4*>(vbytes + vt_chunk_offset(db * 16 + c16, cc * 4 + g));
    };
    u32x4 vbuf[kVDepth];
#pragma unroll
    for (int i = 0; i < kVDepth; ++i) vbuf[i] = fetch_v(i);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MASKED) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = k0 + kb * 16 + 4 * g + i;
            const int row = q_lo + nb * 16 + c16;
            if (key >= T || (CAUSAL && key > row)) sacc[kb][nb][i] = -INFINITY;
          }
    }

    u32x4 pf[2];
    float st[2];
    bool redo = false;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      probs(sacc, nb, mb[nb], pf[nb], st[nb]);
      redo |= !(st[nb] <= 256.f) || m_ref[nb] == -INFINITY;
    }
    if (wave_any(redo)) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float x = sacc[0][nb][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) x = fmaxf(x, sacc[kb][nb][i]);
        const float mn = fmaxf(m_ref[nb], max_across_rows(x) * cs);
        const float alpha = (mn == m_ref[nb]) ? 1.f : fast_exp2(m_ref[nb] - mn);
        const float mb_new = (mn == -INFINITY) ? 0.f : mn;
        probs(sacc, nb, mb_new, pf[nb], st[nb]);
        m_ref[nb] = mn;
        mb[nb] = mb_new;
        l_part[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db][nb] *= alpha;
      }
    }
    l_part[0] += st[0];
    l_part[1] += st[1];

    // O^T += V^T P^T.  V^T fragments (one 16-byte read each) are read kVDepth
    // blocks ahead; the scheduling fences keep each read where it is issued
    // (left alone, the compiler sinks every read to just before its MFMAs and
    // exposes the full LDS latency on each of them).
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const u32x4 vf = vbuf[db % kVDepth];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) o[db][nb] = mfma_f16(vf, pf[nb], o[db][nb]);
      if (db + kVDepth < NDB) vbuf[db % kVDepth] = fetch_v(db + kVDepth);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Key tiles [0, n_int) are fully valid and visible to every row of the
  // workgroup: they take the unmasked step in a branch-free loop, unrolled by
  // two so each stage's LDS offsets are constants.  The remaining (diagonal and
  // ragged) tiles take the masked step.
  // (An interior tile is never the last tile, and its successor is a full
  // tile: the last full tile before a ragged end goes to the tail loop.)
  const int n_int = max(0, CAUSAL ? min((qt * kQTile + 1) / kKeys, T / kKeys - 1) : T / kKeys - 1);
  auto interior_tile = [&](int kt, int stage) __attribute__((always_inline)) {
    // The next tile's loads go out in quarters: before and after each step's
    // score MFMAs.
    if (wave_active) {
      load_k_half(kt + 1, stage ^ 1, 0);
      step(BoolTag<false>{}, smem + stage * TL::kStage, 0, kt * kKeys,
           [&] { load_k_half(kt + 1, stage ^ 1, 1); });
      load_v_half(kt + 1, stage ^ 1, 0);
      step(BoolTag<false>{}, smem + stage * TL::kStage, 1, kt * kKeys + 32,
           [&] { load_v_half(kt + 1, stage ^ 1, 1); });
    } else {
      load_k_tile(kt + 1, stage ^ 1);
      load_v_tile(kt + 1, stage ^ 1);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the next tile landed
    __syncthreads();
  };
  int kt = 0;
  for (; kt + 2 <= n_int; kt += 2) {
    interior_tile(kt, 0);
    interior_tile(kt + 1, 1);
  }
  if (kt < n_int) {
    interior_tile(kt, 0);
    ++kt;
  }
  for (; kt < n_kt; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < n_kt) {
      load_k_tile(kt + 1, stage ^ 1);
      load_v_tile(kt + 1, stage ^ 1);
    }
    if (wave_active) {
      const int t0 = kt * kKeys;
      if (t0 < wave_key_end) step(BoolTag<true>{}, smem + stage * TL::kStage, 0, t0, [] {});
      if (t0 + 32 < wave_key_end) step(BoolTag<true>{}, smem + stage * TL::kStage, 1, t0 + 32, [] {});
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
  }

  // ---- epilogue: stream-2 waves publish O2 / l2 through LDS; stream-1 waves combine ----
  float* xch = reinterpret_cast<float*>(smem);  // [128 rows][XSTRIDE]
  float inv[2], lsum[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    lsum[nb] = sum_across_rows(l_part[nb]);
    inv[nb] = 1.0f / lsum[nb];
  }
  if (a.o1 != nullptr && wave_active) {
    // training forward: this stream's normalised O (fp32) and its log-sum-exp
    // (natural log of the scaled scores; m_ref is in log2 units of s / sqrt(d))
    float* ost = stream == 0 ? a.o1 : a.o2;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int row = q_lo + nb * 16 + c16;
      if (row >= T) continue;
      const size_t r = (tok_base + row) * a.H + h;
      if (g == 0) a.lse[r * 2 + stream] = (m_ref[nb] + log2f(lsum[nb])) * 0.69314718055994531f;
      float* dst = ost + r * DV + g * 4;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        f32x4 t;
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = __fmul_rn(o[db][nb][i], inv[nb]);
        *reinterpret_cast<f32x4*>(dst + db * 16) = t;
      }
    }
  }
  if (stream == 1 && wave_active) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float* dst = xch + (rg * kRows + nb * 16 + c16) * XSTRIDE + g * 4;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        f32x4 t;
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = __fmul_rn(o[db][nb][i], inv[nb]);
        *reinterpret_cast<f32x4*>(dst + db * 16) = t;
      }
    }
  }
  __syncthreads();
  if (stream != 0 || !wave_active) return;
  const float post = 1.0f - a.lambda_init;
  // The lane's weights (channels db*16 + 4g .. +3), all loaded before the first
  // output store: the memory counter also counts stores, so a weight load issued
  // after a store would make its wait cover that store too.
  const bool weighted = a.norm_weight != nullptr;
  f32x4 wv[NDB];
  if (weighted) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[db][i] = a.norm_weight[db * 16 + g * 4 + i];
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float* src = xch + (rg * kRows + nb * 16 + c16) * XSTRIDE + g * 4;
    float ss = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(src + db * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float z = fmaf(-a.lambda, t[i], __fmul_rn(o[db][nb][i], inv[nb]));
        o[db][nb][i] = z;
        ss = fmaf(z, z, ss);
      }
    }
    ss = sum_across_rows(ss);
    const float r = post / sqrtf(ss * (1.0f / DV) + a.eps);
    const int row = q_lo + nb * 16 + c16;
    if (row < T) {
      float* dst = a.out + ((tok_base + row) * a.H + h) * DV + g * 4;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        f32x4 y;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = o[db][nb][i] * r * (weighted ? wv[db][i] : 1.0f);
        *reinterpret_cast<f32x4*>(dst + db * 16) = y;
      }
    }
  }
}

template <int D, int DV>
size_t packed_v_bytes(int B, int T, int H) {
  return (size_t)B * H * ((T + kKeys - 1) / kKeys) * Tile<D, DV>::kVtBytes;
}

template <int D, int DV>
hipError_t launch_typed(const V1Args& a, void* workspace, hipStream_t stream) {
  const long long n_kt = (a.T + kKeys - 1) / kKeys;
  const long long pack_blocks = n_kt * a.B * a.H;
  const long long blocks = (long long)((a.T + kQTile - 1) / kQTile) * a.B * a.H;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL || pack_blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  uint16_t* vp = static_cast<uint16_t*>(workspace);
  hipLaunchKernelGGL((v1_pack_v_kernel<D, DV>), dim3((unsigned)pack_blocks), dim3(DV), 0,
                     stream, a, vp);
  if (a.causal)
    hipLaunchKernelGGL((v1_prefill_kernel<D, DV, true>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, a, vp);
  else
    hipLaunchKernelGGL((v1_prefill_kernel<D, DV, false>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, a, vp);
  return hipGetLastError();
}

}  // namespace

size_t v1_bf16_workspace_bytes(int B, int T, int H, int d, int dv) {
  if (d == 128 && dv == 256) return packed_v_bytes<128, 256>(B, T, H);
  if (d == 64 && dv == 128) return packed_v_bytes<64, 128>(B, T, H);
  return 0;
}

hipError_t launch_v1_bf16(const V1Args& a, void* workspace, hipStream_t stream) {
  if (a.d == 128 && a.dv == 256) return launch_typed<128, 256>(a, workspace, stream);
  if (a.d == 64 && a.dv == 128) return launch_typed<64, 128>(a, workspace, stream);
  return hipErrorInvalidValue;
}

}  // namespace diffattn
