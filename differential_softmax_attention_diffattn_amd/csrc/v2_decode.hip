// DIFF V2 decode step on gfx950: one new query row per sequence against the
// KV cache, for every head pair p:
//     O_j   = softmax_k(q_j . k_{k,kv(j)} * scale) v_{k,kv(j)},  k < cache_len[b]
//     out_p = O_2p - sigmoid(logit_p) * O_2p+1
// The KV heads and cache are those of a standard GQA model, so the step reads
// each cached K/V row once per KV head ("Differential Transformer V2" summary,
// 상세 정리 §2: decoding is memory-bound and V2 does not grow the KV cache).
//
// Split-K.  A workgroup of 8 waves owns (batch entry, cache slice, KVW KV
// heads); wave w takes KV head w % KVW and the (w / KVW)-th part of the slice,
// so with 8 KV heads the workgroup streams whole 2 KiB cache rows (all heads
// of a token) at once.  Each wave walks 32-key chunks: K fragments are loaded
// straight into registers one chunk ahead, V chunks go global->LDS with
// direct-to-LDS buffer loads into a per-wave double buffer and are read back as the
// V^T MFMA operand with the transposing LDS load.  All query heads of the KV
// group (up to 16) share one MFMA column block, so each K/V byte is read once.
// Each wave leaves a partial (O, m, l) per query head; a second kernel merges
// the partials with log-sum-exp weights and applies the pair subtraction.
#include <math.h>

#include <mutex>

#include "device_common.h"
#include "kernels.h"

namespace diffattn {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int kChunk = 32;  // keys per wave step
constexpr float kRescaleLog2 = 8.0f;

// Partial record per (batch, query head, part): O[0..D), m at D, l at D+1, padded
// to a 16-byte multiple so the O stores are aligned.
template <int D>
constexpr int kPartStride = D + 4;

template <int D>
struct DecTile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kBytes = kChunk * kRowBytes;  // one V chunk
  static constexpr int kInstr = kBytes / 1024;       // 1 KiB direct loads per chunk
};

// V rows: 32-byte chunk c of row r at 32-byte position c ^ (r mod n32).
template <int D>
__device__ __forceinline__ int dec_v_offset(int row, int byte_in_row) {
  constexpr int n32 = D / 16;
  const int c32 = byte_in_row >> 5;
  return row * DecTile<D>::kRowBytes + ((c32 ^ (row & (n32 - 1))) << 5) + (byte_in_row & 31);
}

int kv_heads_per_block(int Hkv) {
  if (Hkv % 8 == 0) return 8;
  if (Hkv % 4 == 0) return 4;
  if (Hkv % 2 == 0) return 2;
  return 1;
}

template <int D, int KVW>
__global__ __launch_bounds__(kThreads, 1) void decode_split_kernel(DecodeArgs a) {
  using TL = DecTile<D>;
  constexpr int SUB = kWaves / KVW;  // waves sharing one KV head
  constexpr int NC = D / 32;
  constexpr int NDB = D / 16;
  // The two halves of each wave's V double buffer are separate LDS objects, so
  // the compiler sees that reads of one cannot alias the direct-to-LDS loads in
  // flight into the other and waits only for the loads of the chunk it reads.
  __shared__ __align__(16) uint8_t vbuf0[kWaves][TL::kBytes];
  __shared__ __align__(16) uint8_t vbuf1[kWaves][TL::kBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int c16 = lane & 15;

  const int n_kvg = a.Hkv / KVW;
  const int split = blockIdx.x % a.nsplit;
  const int rest = blockIdx.x / a.nsplit;
  const int kvg = rest % n_kvg;
  const int b = rest / n_kvg;
  const int kv = kvg * KVW + wave % KVW;
  const int sub = wave / KVW;
  const int grp = a.Hq / a.Hkv;
  int n = a.S_max;
  if (a.cache_len != nullptr) n = min(max(a.cache_len[b], 0), a.S_max);
  // this wave's key range: part `sub` of the slice, in whole chunks
  const int s0 = split * a.split_len;
  const int s1 = min(s0 + a.split_len, n);
  const int chunks = s1 > s0 ? (s1 - s0 + kChunk - 1) / kChunk : 0;
  const int per = (chunks + SUB - 1) / SUB;
  const int c_begin = min(sub * per, chunks);
  const int c_end = min(c_begin + per, chunks);

  // Q^T fragment: column c16 = query head kv*grp + c16 (zeros beyond the group)
  u32x4 qf[NC];
  const bool col_valid = c16 < grp;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    qf[c] = col_valid ? ldg128(a.q + ((size_t)b * a.Hq + kv * grp + c16) * D + c * 32 + g * 8)
                      : u32x4{0, 0, 0, 0};

  const size_t row_stride = (size_t)a.Hkv * D;  // elements between consecutive keys
  const uint16_t* kbase = a.k_cache + ((size_t)b * a.S_max * a.Hkv + kv) * D;
  // V: 32-bit byte offsets from the slice start (bounded by one slice)
  const uint16_t* vslice = a.v_cache + (((size_t)b * a.S_max + s0) * a.Hkv + kv) * D;

  auto load_k = [&](int chunk, u32x4 (&kf)[2][NC]) {
    const int base = s0 + chunk * kChunk;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // rows past the end are clamped (their scores are masked), so every load is
      // issued unconditionally and the wait counts stay exact
      const int key = min(base + kb * 16 + c16, s1 - 1);
#pragma unroll
      for (int c = 0; c < NC; ++c) kf[kb][c] = ldg128(kbase + (size_t)key * row_stride + c * 32 + g * 8);
    }
  };
  auto load_v = [&](int chunk, uint8_t* dst) {
    const int base = s0 + chunk * kChunk;
#pragma unroll
    for (int j = 0; j < TL::kInstr; ++j) {
      const int off = j * 1024 + lane * 16;
      const int r = off / TL::kRowBytes;
      const int pos = (off % TL::kRowBytes) >> 4;
      constexpr int n32 = D / 16;
      const int vc = (((pos >> 1) ^ (r & (n32 - 1))) << 1) | (pos & 1);
      const int key = min(base + r, s1 - 1);  // rows past the end are masked (P = 0)
      dma16(vslice, (uint32_t)(((size_t)(key - s0) * row_stride + vc * 8) * 2), dst + j * 1024);
    }
  };

  f32x4 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, mb = 0.f, l_part = 0.f;  // mb: m_ref, or 0 while it is -inf
  const float cs = a.scale * kLog2e;
  const int tr_key = 4 * g + (c16 >> 2);
  const int tr_byte = 8 * (c16 & 3);

  // One 32-key chunk: start the next chunk's loads (K into the other register
  // set, V into the other buffer), then consume this one.  The loads are issued
  // unconditionally (past the wave's last chunk they fetch clamped, valid rows
  // that are never used), so the compiler can count them and waits for exactly
  // the loads each use depends on.
  auto chunk_step = [&](int ci, const u32x4 (&kf)[2][NC], u32x4 (&kn)[2][NC], const uint8_t* vb,
                        uint8_t* vnext) {
    load_k(ci + 1, kn);
    load_v(ci + 1, vnext);
    const int base = s0 + ci * kChunk;

    f32x4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) sacc[kb] = mfma_bf16(kf[kb][c], qf[c], sacc[kb]);
    }
    if (base + kChunk > s1) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (base + kb * 16 + 4 * g + i >= s1) sacc[kb][i] = -INFINITY;
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
        const float e = fast_exp2(fmaf(sacc[kb][i], cs, -mb));
        pv[kb * 4 + i] = e;
        l_part += e;
      }
    const u32x4 pf = u32x4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                           pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const u32x2 lo = lds_read_tr16(vb + dec_v_offset<D>(tr_key, db * 32 + tr_byte));
      const u32x2 hi = lds_read_tr16(vb + dec_v_offset<D>(tr_key + 16, db * 32 + tr_byte));
      o[db] = mfma_bf16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf, o[db]);
    }
    // the buffer read here is refilled by the next step's loads: make sure the
    // reads above have returned first
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  };

  u32x4 ka[2][NC], kb2[2][NC];
  if (c_begin < c_end) {
    load_k(c_begin, ka);
    load_v(c_begin, vbuf0[wave]);
  }
  for (int ci = c_begin; ci < c_end; ci += 2) {
    chunk_step(ci, ka, kb2, vbuf0[wave], vbuf1[wave]);
    if (ci + 1 < c_end) chunk_step(ci + 1, kb2, ka, vbuf1[wave], vbuf0[wave]);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the unused last prefetch has landed

  // ---- this wave's partial (O unnormalised, m in scaled log2 units, l) ----
  const float l_tot = sum_across_rows(l_part);
  if (col_valid) {
    const int part = split * SUB + sub;
    const int nparts = a.nsplit * SUB;
    float* dst = a.partial + (((size_t)b * a.Hq + kv * grp + c16) * nparts + part) * kPartStride<D>;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<f32x4*>(dst + db * 16 + 4 * g) = o[db];
    if (g == 0) {
      dst[D] = m_ref;
      dst[D + 1] = l_tot;
    }
  }
}

// Merge the partials of the two heads an output head subtracts (V2: a pair)
// with log-sum-exp weights, then
// out_p = O_signal(p) - sigmoid(logit_p) * O_noise(p).
// A workgroup owns COLS of the D channels of one output head (D, or a slice of
// 32 when there are many partials, so that a small batch still spreads over
// the device); its 256 threads are COLS columns x 256 / COLS part groups, each
// group summing every (256 / COLS)-th partial, then the groups are added in a
// fixed order.
template <int D, int COLS>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a, int nparts) {
  constexpr int NG = 256 / COLS;
  constexpr int kSlices = D / COLS;
  __shared__ float wts[2][512];
  __shared__ float inv_l[2];
  __shared__ float red[2][NG][COLS];
  // output head p: its block's signal head minus sigmoid-weighted noise head
  // (V2: the pair 2p, 2p + 1)
  const int hp = a.nout;
  const int slice = blockIdx.x % kSlices;
  const int p = (blockIdx.x / kSlices) % hp;
  const int b = blockIdx.x / kSlices / hp;
  const int R = a.ratio;
  const int heads[2] = {(p / R) * (R + 1) + p % R, (p / R) * (R + 1) + R};
  const int t = threadIdx.x;
  const float* src[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
    src[e] = a.partial + (((size_t)b * a.Hq + heads[e]) * nparts) * kPartStride<D>;
  // this thread's channel of parts grp + NG j, up to kPer per head at a time
  // (whole-head workgroups have fewer than 32 parts, a few per thread); the
  // first batch is loaded before the weights are known, so its latency
  // overlaps that of the (m, l) loads
  const int col = t % COLS;
  const int grp = t / COLS;
  const int ch = slice * COLS + col;
  constexpr int kPer = COLS == D ? 4 : 32;
  float ov[2][kPer];
  auto load_batch = [&](int j0) {
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int s = grp + NG * (j0 + j);
        ov[e][j] = s < nparts ? src[e][(size_t)s * kPartStride<D> + ch] : 0.f;
      }
  };
  load_batch(0);
  // weights 2^(m_s - M) / L per part, computed once per head by one wave each;
  // a lane's (m, l) pairs (parts ln + 64 k, at most 512 parts) are all loaded
  // before any is used, so their latencies overlap
  if (t < 2 * kWave) {
    const int e = t / kWave, ln = t % kWave;
    float ms[8], ls[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int s = ln + k * kWave;
      ms[k] = -INFINITY;
      ls[k] = 0.f;
      if (s < nparts) {
        const f32x2 ml = *reinterpret_cast<const f32x2*>(src[e] + s * kPartStride<D> + D);
        ms[k] = ml[0];
        ls[k] = ml[1];
      }
    }
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < 8; ++k) M = fmaxf(M, ms[k]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float L = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int s = ln + k * kWave;
      const float w = (ms[k] == -INFINITY) ? 0.f : fast_exp2(ms[k] - M);
      if (s < nparts) wts[e][s] = w;
      L = fmaf(ls[k], w, L);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
    if (ln == 0) inv_l[e] = L > 0.f ? 1.0f / L : 0.f;
  }
  __syncthreads();
  // four chains per head: part grp + NG j goes to chain j mod 4
  float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int j0 = 0; grp + NG * j0 < nparts; j0 += kPer) {
    if (j0 > 0) load_batch(j0);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int s = grp + NG * (j0 + j);
        if (s < nparts) acc[e][j & 3] = fmaf(ov[e][j], wts[e][s], acc[e][j & 3]);
      }
  }
#pragma unroll
  for (int e = 0; e < 2; ++e) red[e][grp][col] = (acc[e][0] + acc[e][1]) + (acc[e][2] + acc[e][3]);
  __syncthreads();
  if (t >= COLS) return;
  float res[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    float O = 0.f;
#pragma unroll
    for (int k = 0; k < NG; ++k) O += red[e][k][t];
    res[e] = __fmul_rn(O, inv_l[e]);
  }
  const float sg = sigmoid_f32(a.logit[(size_t)b * hp + p]);
  a.out[((size_t)b * hp + p) * D + slice * COLS + t] = f32_to_bf16(fmaf(-sg, res[1], res[0]));
}

template <int D, int KVW>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  const long long blocks = (long long)a.B * (a.Hkv / KVW) * a.nsplit;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_split_kernel<D, KVW>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     stream, a);
  const int nparts = a.nsplit * (kWaves / KVW);
  if (nparts >= 32)
    hipLaunchKernelGGL((decode_combine_kernel<D, 32>), dim3((unsigned)(a.B * a.nout * (D / 32))),
                       dim3(256), 0, stream, a, nparts);
  else
    hipLaunchKernelGGL((decode_combine_kernel<D, D>), dim3((unsigned)(a.B * a.nout)), dim3(256), 0,
                       stream, a, nparts);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  switch (kv_heads_per_block(a.Hkv)) {
    case 8: return launch_typed<D, 8>(a, stream);
    case 4: return launch_typed<D, 4>(a, stream);
    case 2: return launch_typed<D, 2>(a, stream);
    default: return launch_typed<D, 1>(a, stream);
  }
}

}  // namespace

// Compute units of the current device (256 on MI355X), queried once per
// device; 256 when no device can be queried (workspace queries on a host
// without a GPU).
int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static int cached[kMaxDevices] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 256;
  }
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cached[dev] = n;
  }
  return cached[dev];
}

// The longest power-of-two slices (64..65536 keys) that still give one
// workgroup per compute unit (a workgroup's 128 KB of LDS keeps it alone on
// its CU): the whole cache then streams in one round of workgroups, with no
// round boundaries and the fewest partials (measured on B64 S32768 Hkv8:
// 8192-key slices 6.15 TB/s, 2048 6.06, 1024 5.91, 512 5.46).  Small batches
// get slices down to 64 keys (two 32-key chunks per wave) so that they still
// fill the device.  The partial count per (batch, query head) is
// nsplit * (8 / KV heads per workgroup) and stays <= 512.
void decode_split(int B, int S_max, int Hkv, int* split_len, int* nsplit, int* nparts) {
  const int kvw = kv_heads_per_block(Hkv);
  const long long units = (long long)B * (Hkv / kvw);
  const int cus = device_cu_count();
  int len = 65536;
  while (len > 64 && units * ((S_max + len - 1) / len) < cus) len /= 2;
  int ns = S_max > 0 ? (S_max + len - 1) / len : 1;
  const int sub = kWaves / kvw;
  while (ns * sub > 512) {  // bound the partial count (combine kernel weight table)
    len *= 2;
    ns = (S_max + len - 1) / len;
  }
  *split_len = len;
  *nsplit = ns;
  *nparts = ns * sub;
}

hipError_t launch_v2_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_d<128>(a, stream);
  if (a.d == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

// Partial results of the decode entry point that allocates nothing
// (diffattn_v2_decode_noalloc).  Every GPU the library runs on holds its own
// copy until the process ends, and every such call on that GPU uses it, so
// calls that overlap on one GPU race.  The split kernel writes every record
// the combine kernel reads (empty slices included), so nothing in it needs to
// start at zero.  Host code never uses the array's name, which is only a
// host-side stand-in: it uses the device address looked up below.
namespace {
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
}  // namespace

size_t decode_noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

void* decode_noalloc_scratch(hipError_t* err) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with this device current
    if (e != hipSuccess || p == nullptr) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    ptrs[dev] = p;
  }
  *err = hipSuccess;
  return ptrs[dev];
}

}  // namespace diffattn
