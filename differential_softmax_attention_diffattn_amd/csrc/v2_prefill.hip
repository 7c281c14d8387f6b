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
// Work decomposition: a workgroup of 8 waves (two per SIMD) owns a tile of
// query rows and PW consecutive head pairs of one KV head.  Each wave owns one
// pair and 16 rows, i.e. two 16-column MFMA blocks (even head, odd head) that
// share every K and V fragment it reads.  Every K/V tile staged in LDS serves
// all 2*PW query heads of the workgroup.
//
// Per 32-key step a wave computes S^T = K Q^T on 16x16x32 bf16 MFMA (keys on
// the M side, query columns on N), so each lane holds one query column: the
// softmax statistics are per lane, P^T feeds the second MFMA directly as its B
// operand, and O^T = V^T P^T accumulates with the head dim on M.  K and V
// tiles arrive by direct-to-LDS loads, both row-major with XOR-swizzled
// chunks; the V^T operand is read with the transposing LDS load.  Both heads of
// a pair sit in the same lane (same row, same d), so the sigmoid-weighted
// subtraction happens in registers and only h*d bf16 columns are written.
// Rescaling of O is lazy: the reference maximum only moves when a column's
// maximum grows by more than 2^8, which keeps P <= 256 (exact in O / l).
#include <math.h>

#include "device_common.h"
#include "kernels.h"
#include "varlen.h"

namespace diffattn {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int kRows = 16;   // query rows per wave
constexpr int kKeys = 64;   // keys per staged KV tile
constexpr int kVDepth = 2;  // V^T fragments in flight during P.V
constexpr float kRescaleLog2 = 8.0f;

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

template <int D>
struct Tile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;             // 16-byte chunks per row
  static constexpr int kTileBytes = kKeys * kRowBytes;
  static constexpr int kStage = 2 * kTileBytes;     // K then V
  static constexpr int kInstr = kTileBytes / 1024;  // 1 KiB direct loads per tile
};

// K rows: 16-byte chunk c of row r sits at chunk position c ^ (r mod nchunks).
template <int D>
__device__ __forceinline__ int k_offset(int row, int chunk) {
  return row * Tile<D>::kRowBytes + ((chunk ^ (row & (Tile<D>::kChunks - 1))) << 4);
}
// V rows: 32-byte chunk c of row r sits at 32-byte position c ^ (r mod n32), so
// the 16 rows one transposing read touches spread over the LDS banks.
template <int D>
__device__ __forceinline__ int v_offset(int row, int byte_in_row) {
  constexpr int n32 = D / 16;
  const int c32 = byte_in_row >> 5;
  return row * Tile<D>::kRowBytes + ((c32 ^ (row & (n32 - 1))) << 5) + (byte_in_row & 31);
}

// SHARED (grouped variant with ratio + 1 dividing 2 PW): each wave computes
// the two consecutive query heads 2pp, 2pp + 1 once, as for V2, and the
// subtraction happens in the epilogue: waves holding a noise head publish its
// normalised output through LDS, and every signal head subtracts its block's
// noise head from there or from its own registers.  Otherwise each wave
// computes an output head's signal and noise head itself (V2: the pair).
template <int D, int PW, bool CAUSAL, bool SHARED>
__global__ __launch_bounds__(kThreads, 1) void v2_prefill_kernel(V2Args a) {
  using TL = Tile<D>;
  constexpr int QSUB = kWaves / PW;  // 16-row groups per workgroup
  constexpr int QTILE = kRows * QSUB;
  constexpr int NC = D / 32;   // k-chunks of Q K^T
  constexpr int NDB = D / 16;  // 16-row blocks of O^T
  static_assert(TL::kInstr % kWaves == 0, "tile loads must split evenly over the waves");

  // Two pipeline stages as two separate LDS objects: the compiler then knows
  // the transposing reads of one stage cannot alias the direct-to-LDS loads in
  // flight into the other, and does not wait for those loads before each read.
  __shared__ __align__(16) uint8_t smem0[TL::kStage];
  __shared__ __align__(16) uint8_t smem1[TL::kStage];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int c16 = lane & 15;

  // ---- block -> (sequence, query tile, pair group) ----
  // Sequence-major: the query tiles of a sequence are numbered consecutively,
  // longest (last) tile first, and the pair groups of a tile are adjacent.  With
  // one pair group per KV head and 8 of them, blocks of one KV head land on one
  // XCD and that XCD's CUs work through the tiles of one sequence together,
  // sharing its K/V tiles in L2.  Packed batches number the tiles by slots
  // (varlen.h): a search over cu_seqlens by the whole wave finds the sequence, and the
  // blocks of empty slots exit.
  const int n_hg = SHARED ? a.Hq / 2 / PW : a.nout / PW;
  const int hg = blockIdx.x % n_hg;
  const int t = blockIdx.x / n_hg;
  int tok0, L, qt;
  if (a.cu_seqlens != nullptr) {
    // every sequence within one query tile: tile t is sequence t (no slots)
    const bool one_tile = a.max_seqlen <= QTILE;
    const int seq = one_tile ? t : slot_sequence_wave(a.cu_seqlens, a.nseq, t, QTILE);
    tok0 = a.cu_seqlens[seq];
    L = a.cu_seqlens[seq + 1] - tok0;
    const int nt = (L + QTILE - 1) / QTILE;
    const int tile = one_tile ? 0 : (int)(t - slot_start(a.cu_seqlens, seq, QTILE));
    if (tile >= nt) return;  // an empty slot: uniform over the block
    qt = nt - 1 - tile;
  } else {
    const int nt = (a.T + QTILE - 1) / QTILE;
    const int seq = t / nt;
    qt = nt - 1 - (t - seq * nt);
    tok0 = seq * a.T;
    L = a.T;
  }

  // output head p subtracts its block's noise head from its signal head (V2:
  // blocks of two, the pair 2p, 2p + 1); the PW output heads of a workgroup
  // lie in one GQA group (the launch picks PW so)
  const int nout = a.nout;
  const int group = a.Hq / a.Hkv;
  const int R = a.ratio;
  const int p = hg * PW + (wave % PW);
  // the wave's two query heads: SHARED, the pair 2p, 2p + 1 (2p is a signal
  // head: blocks start at even heads and end with their noise head); else the
  // signal and noise head of output head p
  const int head_sig = SHARED ? 2 * p : (p / R) * (R + 1) + p % R;
  const int head_noise = SHARED ? 2 * p + 1 : (p / R) * (R + 1) + R;
  const int kv = SHARED ? (hg * PW * 2) / group : (((hg * PW) / R) * (R + 1)) / group;
  // output-head index of a signal query head j
  auto out_index = [&](int j) { return (j / (R + 1)) * R + j % (R + 1); };
  const bool odd_is_noise = SHARED && (head_noise % (R + 1) == R);
  const int q_lo = qt * QTILE + (wave / PW) * kRows;
  const bool wave_active = q_lo < L;

  const int q_end_block = min(qt * QTILE + QTILE, L);
  const int n_kt = CAUSAL ? (q_end_block - 1) / kKeys + 1 : (L + kKeys - 1) / kKeys;
  const int wave_key_end = CAUSAL ? min(q_lo + kRows, L) : L;

  // ---- Q^T fragments (B operand): block 0 = even head, block 1 = odd head ----
  // Q is pre-multiplied by scale * log2(e) (rounded to bf16), so the score MFMA
  // yields log2-domain logits directly.
  const float cs = a.scale * kLog2e;
  const int row = q_lo + c16;
  // Every load of the prologue goes out before any of its results is used:
  // rows past the sequence end read its last row (L >= 1 here) and are zeroed
  // when scaled, after the first tile's loads have been issued.  (Loading and
  // scaling row by row under `row < L` made each load wait for the one before.)
  const int rowc = min(row, L - 1);
  u32x4 qf[2][NC];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qf[nb][c] = ldg128(a.q + ((size_t)(tok0 + rowc) * a.Hq + (nb ? head_noise : head_sig)) * D +
                         c * 32 + g * 8);
  // the pair's coefficient logit for this lane's row, fetched now so its load
  // latency is not paid at the end of the key loop
  const float lgv = a.logit[(size_t)(tok0 + rowc) * nout + (SHARED ? out_index(head_sig) : p)];
  const float lgv_odd =
      (SHARED && !odd_is_noise) ? a.logit[(size_t)(tok0 + rowc) * nout + out_index(head_noise)] : 0.f;

  // ---- direct-to-LDS tile loads (K and V rows, swizzled) ----
  // Each lane's chunks inside a tile are fixed; keep them as 32-bit element
  // offsets from the tile's first key and move the tile base in scalar
  // registers.  Rows past the sequence end are clamped on the ragged last tile.
  const size_t kv_stride = (size_t)a.Hkv * D;  // elements between consecutive tokens
  const uint16_t* kbase_g = a.k + ((size_t)tok0 * a.Hkv + kv) * D;
  const uint16_t* vbase_g = a.v + ((size_t)tok0 * a.Hkv + kv) * D;
  constexpr int NJ = TL::kInstr / kWaves;
  // A lane's LDS bytes in its j-th load of a tile lie kJRows rows below those of
  // its first load; kJRows is a multiple of both swizzle periods, so the chunk
  // it fetches is the same and the j-th global offset differs by a uniform
  // kJRows rows (added to the scalar base).
  constexpr int kJRows = kWaves * 1024 / TL::kRowBytes;
  static_assert(kJRows % TL::kChunks == 0 && kJRows % (D / 16) == 0, "loads must repeat the swizzle");
  auto lane_chunks = [&](int j, int& r, int& kc, int& vc) {
    const int off = (wave + j * kWaves) * 1024 + lane * 16;  // LDS byte offset this lane fills
    r = off / TL::kRowBytes;
    const int pos = (off % TL::kRowBytes) >> 4;
    kc = pos ^ (r & (TL::kChunks - 1));  // K: position pos holds chunk pos ^ (r mod nchunks)
    constexpr int n32 = D / 16;          // V: 32-byte position pos/2 holds (pos/2) ^ (r mod n32)
    vc = (((pos >> 1) ^ (r & (n32 - 1))) << 1) | (pos & 1);
  };
  uint32_t k_lane_off, v_lane_off;  // bytes, first load of a tile
  {
    int r, kc, vc;
    lane_chunks(0, r, kc, vc);
    k_lane_off = (uint32_t)((r * kv_stride + kc * 8) * 2);
    v_lane_off = (uint32_t)((r * kv_stride + vc * 8) * 2);
  }
  auto load_tiles = [&](int kt, uint8_t* base) {
    const size_t tile = (size_t)kt * kKeys * kv_stride;
    if ((kt + 1) * kKeys <= L) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int blk = wave + j * kWaves;
        const size_t jrow = tile + (size_t)j * kJRows * kv_stride;
        dma16(kbase_g + jrow, k_lane_off, base + blk * 1024);
        dma16(vbase_g + jrow, v_lane_off, base + TL::kTileBytes + blk * 1024);
      }
    } else {  // ragged last tile: clamp rows past the sequence end (they are masked)
      // (offsets relative to the tile's first key, so they stay within 32 bits
      // for any sequence length)
      const int last = L - 1 - kt * kKeys;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int blk = wave + j * kWaves;
        int r, kc, vc;
        lane_chunks(j, r, kc, vc);
        const size_t rr = (size_t)min(r, last);
        dma16(kbase_g + tile, (uint32_t)((rr * kv_stride + kc * 8) * 2), base + blk * 1024);
        dma16(vbase_g + tile, (uint32_t)((rr * kv_stride + vc * 8) * 2),
              base + TL::kTileBytes + blk * 1024);
      }
    }
  };

  load_tiles(0, smem0);
  // Q pre-multiplied by scale * log2(e) (rounded to bf16); rows past the end zeroed
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qf[nb][c] = row < L ? scale_bf16x8(qf[nb][c], cs) : u32x4{0, 0, 0, 0};
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): direct-to-LDS loads landed
  __syncthreads();

  f32x4 o[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) o[db][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Softmax state per column block (log2 units): m_ref is the reference
  // maximum, -inf until the first key; mb is m_ref with -inf replaced by 0, the
  // value subtracted before exp2; sinit = {-mb x 4} starts every score MFMA
  // chain, so the accumulators come out as S*scale*log2(e) - mb.
  float m_ref[2] = {-INFINITY, -INFINITY}, mb[2] = {0.f, 0.f}, l_part[2] = {0.f, 0.f};
  f32x4 sinit[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};

  // Per-lane LDS offsets, fixed for the whole key loop.  K operand: row c16 of
  // a 16-key block, chunk 4c + g.  V^T operand (transposing read): lane j of a
  // 16-lane row supplies key 4g + j/4 and d 4(j%4) of 32-byte column block db.
  // Offsets of the 32-key step and the upper 16 keys are added as immediates.
  const int tr_key = 4 * g + (c16 >> 2);
  const int tr_byte = 8 * (c16 & 3);
  int k_ofs[NC], v_ofs[NDB];
#pragma unroll
  for (int c = 0; c < NC; ++c) k_ofs[c] = k_offset<D>(c16, c * 4 + g);
#pragma unroll
  for (int db = 0; db < NDB; ++db) v_ofs[db] = v_offset<D>(tr_key, db * 32 + tr_byte);

  // P for one column block from its two score accumulators, minus `shift`:
  // packed bf16 fragment plus the per-lane sum of the rounded values.
  auto probs = [&](const f32x4 (&sacc)[2][2], int nb, float shift, u32x4& pf, float& st) {
    float pv[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[kb * 4 + i] = fast_exp2(sacc[kb][nb][i] - shift);
    pf = u32x4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
               pack_bf16x2(pv[6], pv[7])};
    st = sum_bf16x8(pf, 0.f);
  };

  // One 32-key step; MASKED adds the causal / ragged mask (only the key tiles
  // on the diagonal or at the sequence end need it).
  //
  // Lazy rescaling, checked after the fact: P = 2^(s - mb) is computed with the
  // current reference; if some lane's eight values sum past 2^8 (so some P may
  // exceed 2^8) or no reference exists yet, the wave takes the rare path: the
  // column maxima are computed, the reference moves up to them, O and l are
  // rescaled and P is recomputed (now <= 1).  Otherwise every P <= 2^8, which
  // bf16 P and the fp32 O / l accumulators carry without loss of range.
  auto step = [&](auto masked, const uint8_t* k_lds, const uint8_t* v_lds, int cc, int k0, auto mid) {
    constexpr bool MASKED = decltype(masked)::value;
    // S^T = K Q^T - mb: 2 key blocks x 2 column blocks
    f32x4 sacc[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) sacc[kb][nb] = sinit[nb];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(
            k_lds + k_ofs[c] + (cc * 32 + kb * 16) * TL::kRowBytes);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) sacc[kb][nb] = mfma_bf16(kf, qf[nb][c], sacc[kb][nb]);
      }
    }
    mid();  // work to issue between the score MFMAs and the softmax
    // the first V^T fragments (transposing reads of the row-major V tile) go
    // out before the softmax
    auto fetch_v = [&](int db) {
      const uint8_t* vp = v_lds + v_ofs[db] + cc * 32 * TL::kRowBytes;
      const u32x2 lo = lds_read_tr16(vp);
      const u32x2 hi = lds_read_tr16(vp + 16 * TL::kRowBytes);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    u32x4 vbuf[kVDepth];
#pragma unroll
    for (int i = 0; i < kVDepth; ++i) vbuf[i] = fetch_v(i);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MASKED) {  // same rows for both heads of the pair
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + kb * 16 + 4 * g + i;
          if (key >= L || (CAUSAL && key > row)) {
            sacc[kb][0][i] = -INFINITY;
            sacc[kb][1][i] = -INFINITY;
          }
        }
    }

    u32x4 pf[2];
    float st[2];
    bool redo = false;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      probs(sacc, nb, 0.f, pf[nb], st[nb]);
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
        const float mn = fmaxf(m_ref[nb], max_across_rows(x) + mb[nb]);
        const float alpha = (mn == m_ref[nb]) ? 1.f : fast_exp2(m_ref[nb] - mn);
        const float mb_new = (mn == -INFINITY) ? 0.f : mn;
        probs(sacc, nb, mb_new - mb[nb], pf[nb], st[nb]);
        m_ref[nb] = mn;
        mb[nb] = mb_new;
        sinit[nb] = f32x4{-mb_new, -mb_new, -mb_new, -mb_new};
        l_part[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db][nb] *= alpha;
      }
    }
    l_part[0] += st[0];
    l_part[1] += st[1];

    // O^T += V^T P^T.  V^T fragments are read kVDepth blocks ahead; the
    // scheduling fences keep each read where it is issued (left alone, the
    // compiler sinks every read to just before its MFMAs and exposes the full
    // LDS latency on each of them).
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const u32x4 vf = vbuf[db % kVDepth];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) o[db][nb] = mfma_bf16(vf, pf[nb], o[db][nb]);
      if (db + kVDepth < NDB) vbuf[db % kVDepth] = fetch_v(db + kVDepth);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // SHARED epilogue.  xch holds, per row group and block of the workgroup,
  // the block's normalised noise-head output [16 rows][D] (fp32, padded rows).
  auto shared_epilogue = [&]() __attribute__((always_inline)) {
    constexpr int XS = D + 4;
    constexpr int kBlocks = 2 * PW / 4 > 0 ? 2 * PW / 4 : 1;  // blocks (>= 4 heads) in 2 PW heads
    __shared__ __align__(16) float xch[QSUB][kBlocks][kRows * XS];
    const int rg = wave / PW;
    const int head0 = 2 * hg * PW;  // first query head of the workgroup
    const float l_e = sum_across_rows(l_part[0]);
    const float l_o = sum_across_rows(l_part[1]);
    const float inv_e = 1.0f / l_e;
    const float inv_o = 1.0f / l_o;
    if (wave_active && odd_is_noise) {
      float* dst = &xch[rg][(head_noise - head0) / (R + 1)][c16 * XS + g * 4];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        f32x4 t;
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = __fmul_rn(o[db][1][i], inv_o);
        *reinterpret_cast<f32x4*>(dst + db * 16) = t;
      }
    }
    __syncthreads();
    if (!wave_active || row >= L) return;
    const size_t tok = (size_t)(tok0 + row);
    if (a.o_heads != nullptr) {  // training forward: every head once
      if (g == 0) {
        a.lse[tok * a.Hq + head_sig] = (mb[0] + log2f(l_e)) * 0.69314718055994531f;
        a.lse[tok * a.Hq + head_noise] = (mb[1] + log2f(l_o)) * 0.69314718055994531f;
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const float inv = nb ? inv_o : inv_e;
        uint16_t* dst = a.o_heads + (tok * a.Hq + (nb ? head_noise : head_sig)) * D + g * 4;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          *reinterpret_cast<u32x2*>(dst + db * 16) =
              u32x2{pack_bf16x2(o[db][nb][0] * inv, o[db][nb][1] * inv),
                    pack_bf16x2(o[db][nb][2] * inv, o[db][nb][3] * inv)};
      }
    }
    // the even head always subtracts its block's noise head: the odd head of
    // this wave, or published by another wave
    const int noise_e = (head_sig / (R + 1)) * (R + 1) + R;
    const float* xn = &xch[rg][(noise_e - head0) / (R + 1)][c16 * XS + g * 4];
    const float sg_e = sigmoid_f32(lgv);
    const float sg_o = sigmoid_f32(lgv_odd);
    uint16_t* dst_e = a.out + (tok * nout + out_index(head_sig)) * D + g * 4;
    uint16_t* dst_o = a.out + (tok * nout + out_index(head_noise)) * D + g * 4;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      f32x4 n4;
      if (odd_is_noise) {
#pragma unroll
        for (int i = 0; i < 4; ++i) n4[i] = __fmul_rn(o[db][1][i], inv_o);
      } else {
        n4 = *reinterpret_cast<const f32x4*>(xn + db * 16);
      }
      float r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = fmaf(-sg_e, n4[i], __fmul_rn(o[db][0][i], inv_e));
      *reinterpret_cast<u32x2*>(dst_e + db * 16) = u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
      if (!odd_is_noise) {
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = fmaf(-sg_o, n4[i], __fmul_rn(o[db][1][i], inv_o));
        *reinterpret_cast<u32x2*>(dst_o + db * 16) = u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
      }
    }
  };

  // Key tiles [0, n_int) are fully valid and visible to every row of the
  // workgroup: they take the unmasked step in a branch-free loop, unrolled by
  // two so each stage is a fixed LDS object.  The remaining (diagonal and
  // ragged) tiles take the masked step with the stage chosen at run time.
  const int q_lo_block = qt * QTILE;
  const int n_int = max(0, CAUSAL ? min((q_lo_block + 1) / kKeys, L / kKeys - 1) : L / kKeys - 1);
  // Quarters of a full tile's loads (K or V, first or second half of this
  // wave's share), spread through a tile's compute: all eight waves issuing a
  // whole tile at once stall for hundreds of cycles at the load issue.
  constexpr int kHalf = (NJ + 1) / 2;
  auto load_quarter = [&](int kt, uint8_t* base, int which, int half) __attribute__((always_inline)) {
    const size_t tile = (size_t)kt * kKeys * kv_stride;
#pragma unroll
    for (int j = half * kHalf; j < min((half + 1) * kHalf, NJ); ++j) {
      const int blk = wave + j * kWaves;
      const size_t jrow = tile + (size_t)j * kJRows * kv_stride;
      if (which == 0)
        dma16(kbase_g + jrow, k_lane_off, base + blk * 1024);
      else
        dma16(vbase_g + jrow, v_lane_off, base + TL::kTileBytes + blk * 1024);
    }
  };
  // An interior tile is never the last one and its successor is full (the last
  // full tile before a ragged end goes to the tail loop).
  auto interior_tile = [&](int kt, const uint8_t* k_lds, uint8_t* next) {
    if (wave_active) {
      const uint8_t* v_lds = k_lds + TL::kTileBytes;
      load_quarter(kt + 1, next, 0, 0);
      step(BoolTag<false>{}, k_lds, v_lds, 0, kt * kKeys, [&] { load_quarter(kt + 1, next, 0, 1); });
      load_quarter(kt + 1, next, 1, 0);
      step(BoolTag<false>{}, k_lds, v_lds, 1, kt * kKeys + 32, [&] { load_quarter(kt + 1, next, 1, 1); });
    } else {
      load_tiles(kt + 1, next);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the next tile landed
    __syncthreads();
  };
  int kt = 0;
  for (; kt + 2 <= n_int; kt += 2) {
    interior_tile(kt, smem0, smem1);
    interior_tile(kt + 1, smem1, smem0);
  }
  if (kt < n_int) {
    interior_tile(kt, smem0, smem1);
    ++kt;
  }
  for (; kt < n_kt; ++kt) {
    uint8_t* cur = (kt & 1) ? smem1 : smem0;
    uint8_t* next = (kt & 1) ? smem0 : smem1;
    if (kt + 1 < n_kt) load_tiles(kt + 1, next);
    if (wave_active) {
      const uint8_t* v_lds = cur + TL::kTileBytes;
      const int t0 = kt * kKeys;
      if (t0 < wave_key_end) step(BoolTag<true>{}, cur, v_lds, 0, t0, [] {});
      if (t0 + 32 < wave_key_end) step(BoolTag<true>{}, cur, v_lds, 1, t0 + 32, [] {});
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
  }

  if constexpr (SHARED) {
    shared_epilogue();
    return;
  }
  if (!wave_active) return;

  // ---- epilogue: normalise, pair subtraction, bf16 store ----
  const float l_e = sum_across_rows(l_part[0]);
  const float l_o = sum_across_rows(l_part[1]);
  const float inv_e = 1.0f / l_e;
  const float inv_o = 1.0f / l_o;
  if (row < L && a.o_heads != nullptr) {
    // training forward: per-head outputs and natural-log log-sum-exp of the
    // scaled scores (the accumulators hold log2-domain values minus mb)
    const size_t tok = (size_t)(tok0 + row);
    if (g == 0) {
      a.lse[tok * a.Hq + head_sig] = (mb[0] + log2f(l_e)) * 0.69314718055994531f;
      a.lse[tok * a.Hq + head_noise] = (mb[1] + log2f(l_o)) * 0.69314718055994531f;
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float inv = nb ? inv_o : inv_e;
      uint16_t* dst = a.o_heads + (tok * a.Hq + (nb ? head_noise : head_sig)) * D + g * 4;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *reinterpret_cast<u32x2*>(dst + db * 16) =
            u32x2{pack_bf16x2(o[db][nb][0] * inv, o[db][nb][1] * inv),
                  pack_bf16x2(o[db][nb][2] * inv, o[db][nb][3] * inv)};
    }
  }
  if (row < L) {
    const size_t tok = (size_t)(tok0 + row);
    const float sg = sigmoid_f32(lgv);
    uint16_t* dst = a.out + (tok * nout + p) * D + g * 4;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      float r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ev = __fmul_rn(o[db][0][i], inv_e);
        const float od = __fmul_rn(o[db][1][i], inv_o);
        r[i] = fmaf(-sg, od, ev);
      }
      *reinterpret_cast<u32x2*>(dst + db * 16) =
          u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
    }
  }
}

template <int D, int PW, bool SHARED>
hipError_t launch_typed(const V2Args& a, hipStream_t stream) {
  constexpr int QTILE = kRows * (kWaves / PW);
  // query tiles: B x ceil(T / QTILE) for padded batches, the tile slots of
  // varlen.h for packed ones
  const long long tiles = a.cu_seqlens == nullptr ? (long long)((a.T + QTILE - 1) / QTILE) * a.nseq
                          : a.max_seqlen <= QTILE ? (long long)a.nseq
                                                  : slot_count(a.N, a.nseq, a.max_seqlen, QTILE);
  const long long blocks = tiles * (SHARED ? a.Hq / 2 / PW : a.nout / PW);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.causal)
    hipLaunchKernelGGL((v2_prefill_kernel<D, PW, true, SHARED>), dim3((unsigned)blocks),
                       dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((v2_prefill_kernel<D, PW, false, SHARED>), dim3((unsigned)blocks),
                       dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const V2Args& a, hipStream_t stream) {
  const int group = a.Hq / a.Hkv;
  const int R = a.ratio;
  // grouped variant whose blocks of ratio + 1 heads tile a workgroup's 2 PW
  // query heads: every head computed once (SHARED)
  if (R > 1 && (R + 1) % 2 == 0 && a.o_heads == nullptr) {
    const int pairs_per_group = group / 2;
    if (pairs_per_group % 4 == 0 && 8 % (R + 1) == 0) return launch_typed<D, 4, true>(a, stream);
    if (pairs_per_group % 2 == 0 && 4 % (R + 1) == 0) return launch_typed<D, 2, true>(a, stream);
  }
  // otherwise a workgroup's PW output heads must share one GQA group
  const int out_per_group = group / (R + 1) * R;
  if (out_per_group % 4 == 0) return launch_typed<D, 4, false>(a, stream);
  if (out_per_group % 2 == 0) return launch_typed<D, 2, false>(a, stream);
  return launch_typed<D, 1, false>(a, stream);
}

}  // namespace

hipError_t launch_v2_prefill(const V2Args& a, hipStream_t stream) {
  if (a.d == 128) return launch_d<128>(a, stream);
  if (a.d == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace diffattn
