// The two projections either side of the V2 attention ("Differential
// Transformer V2" summary, 상세 정리 §1 and §7):
//  * lambda_proj_kernel: the per-token, per-pair coefficient logits projected
//    from the layer input, logits[n, p] = sum_c x[n, c] w[p, c] (the sigmoid
//    is applied where the coefficient is used, in the attention epilogue).
//    A skinny GEMM (h <= 64 outputs), bound by reading X once from HBM.
//  * gemm_tn_kernel: the output projection on the h*d columns left after the
//    subtraction, y[m, n] = sum_k a[m, k] w[n, k] (weights one row per output
//    feature, so both operands are contiguous along k).  An MFMA GEMM.
// bf16 inputs, fp32 accumulation (16x16x32 MFMA).
#include "device_common.h"
#include "kernels.h"

namespace diffattn {
namespace {

// ---------------------------------------------------------------------------
// Coefficient logits.  A workgroup owns 32 tokens (two 16-row blocks) and all
// NB * 16 outputs; its 4 waves split d_model into quarters and their partial
// sums are added in LDS (fixed order).  Each lane reads 32 contiguous bytes of
// a row per 64-wide k slab (two MFMA k-steps): the MFMA's k order is permuted
// the same way for X and W, so four lanes cover one 128-byte line of a row.
// ---------------------------------------------------------------------------
constexpr int kProjRowBlocks = 2;
constexpr int kProjTokens = kProjRowBlocks * 16;
constexpr int kProjWaves = 4;

template <int NB>
__global__ __launch_bounds__(kProjWaves * kWave) void lambda_proj_kernel(LambdaProjArgs a) {
  __shared__ f32x4 part[kProjWaves - 1][kProjRowBlocks][NB][kWave];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const long long tok0 = (long long)blockIdx.x * kProjTokens;
  const int D = a.d_model;
  const int kq = D / kProjWaves;  // this wave's quarter of d_model
  const uint16_t* xr[kProjRowBlocks];
#pragma unroll
  for (int mb = 0; mb < kProjRowBlocks; ++mb) {
    const long long row = min(tok0 + mb * 16 + c16, a.N - 1);  // ragged tail: clamp
    xr[mb] = a.x + row * D + wave * kq + g * 16;
  }
  const uint16_t* wr[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) wr[nb] = a.w + (size_t)(nb * 16 + c16) * D + wave * kq + g * 16;
  f32x4 acc[kProjRowBlocks][NB];
#pragma unroll
  for (int mb = 0; mb < kProjRowBlocks; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < kq; k += 64) {
    u32x4 xa[kProjRowBlocks][2], wb[NB][2];
#pragma unroll
    for (int mb = 0; mb < kProjRowBlocks; ++mb) {
      xa[mb][0] = ldg128(xr[mb] + k);
      xa[mb][1] = ldg128(xr[mb] + k + 8);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      wb[nb][0] = ldg128(wr[nb] + k);
      wb[nb][1] = ldg128(wr[nb] + k + 8);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int mb = 0; mb < kProjRowBlocks; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = mfma_bf16(xa[mb][s], wb[nb][s], acc[mb][nb]);
  }
  if (wave > 0) {
#pragma unroll
    for (int mb = 0; mb < kProjRowBlocks; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) part[wave - 1][mb][nb][lane] = acc[mb][nb];
  }
  __syncthreads();
  if (wave > 0) return;
  // C layout: element i of block (mb, nb) is token 16 mb + 4 g + i, output 16 nb + c16
  const int H = NB * 16;
#pragma unroll
  for (int mb = 0; mb < kProjRowBlocks; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4 t = acc[mb][nb];
#pragma unroll
      for (int w = 0; w < kProjWaves - 1; ++w) {
        const f32x4 p = part[w][mb][nb][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] += p[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long long row = tok0 + mb * 16 + 4 * g + i;
        if (row < a.N) a.logits[row * H + nb * 16 + c16] = t[i];
      }
    }
}

// ---------------------------------------------------------------------------
// Output projection: C[M, N] = A[M, K] * W[N, K]^T.  A workgroup of 8 waves
// owns a 256 x 256 tile of C, a wave 128 x 64 (8 x 4 MFMA blocks); A and W
// tiles of 256 rows x 64 k (32 KB each) go global -> LDS by direct loads,
// double-buffered.  LDS rows are 128 bytes; the 16-byte chunk c of row r sits
// at position c ^ ((r >> 1) & 7), so the 16 rows an MFMA operand read touches
// (two rows per 256-byte bank window) land in 16 distinct bank groups.
// Tiles are numbered so that each XCD (workgroups are dealt to the 8 XCDs
// round-robin) works on a band of 8 row tiles across all column tiles: the
// band's A rows and the W tiles are shared in that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int kGemmTile = 256;
constexpr int kGemmK = 64;
constexpr int kGemmWaves = 8;
constexpr int kGemmTileBytes = kGemmTile * kGemmK * 2;
constexpr int kGemmGroupM = 8;
constexpr int kXcds = 8;

__device__ __forceinline__ int gemm_lds_offset(int row, int chunk) {
  return row * (kGemmK * 2) + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// rows r0 .. r0+255 of a [rows, K] bf16 matrix (rows >= n_valid clamped), k
// columns k0 .. k0+63, into the swizzled tile: 32 loads of 1 KiB, 4 per wave.
__device__ __forceinline__ void gemm_load_tile(const uint16_t* base, long long K, long long r0,
                                               long long n_valid, int k0, uint8_t* lds, int wave,
                                               int lane) {
  const long long rb = min(r0, n_valid - 1);  // wave-uniform base row
#pragma unroll
  for (int j = 0; j < kGemmTileBytes / 1024 / kGemmWaves; ++j) {
    const int blk = wave + j * kGemmWaves;
    const int off = blk * 1024 + lane * 16;  // LDS byte this lane fills
    const int r = off >> 7;                  // 128-byte rows
    const int pos = (off & 127) >> 4;
    const int lc = pos ^ ((r >> 1) & 7);  // logical chunk stored at that position
    const long long row = min(r0 + r, n_valid - 1);
    dma16(base + rb * K + k0, (uint32_t)(((row - rb) * K + lc * 8) * 2), lds + blk * 1024);
  }
}

__global__ __launch_bounds__(kGemmWaves * kWave, 1) void gemm_tn_kernel(GemmArgs a) {
  __shared__ __align__(16) uint8_t sa0[kGemmTileBytes];
  __shared__ __align__(16) uint8_t sb0[kGemmTileBytes];
  __shared__ __align__(16) uint8_t sa1[kGemmTileBytes];
  __shared__ __align__(16) uint8_t sb1[kGemmTileBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves of 128 x 64
  const int tiles_m = (int)((a.M + kGemmTile - 1) / kGemmTile);
  const int tiles_n = (int)((a.N + kGemmTile - 1) / kGemmTile);
  const int ntiles = tiles_m * tiles_n;
  // workgroup -> tile: consecutive tile numbers on one XCD, grouped by 8 row tiles
  int pid = blockIdx.x;
  if (ntiles % kXcds == 0) pid = (blockIdx.x % kXcds) * (ntiles / kXcds) + blockIdx.x / kXcds;
  const int per_group = kGemmGroupM * tiles_n;
  const int group = pid / per_group;
  const int first_m = group * kGemmGroupM;
  const int gm = min(tiles_m - first_m, kGemmGroupM);
  const int tm = first_m + (pid % per_group) % gm;
  const int tn = (pid % per_group) / gm;
  const long long m0 = (long long)tm * kGemmTile;
  const long long n0 = (long long)tn * kGemmTile;
  const int nk = (int)(a.K / kGemmK);

  f32x4 acc[8][4];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load = [&](int kt, uint8_t* la, uint8_t* lb) {
    gemm_load_tile(a.a, a.K, m0, a.M, kt * kGemmK, la, wave, lane);
    gemm_load_tile(a.w, a.K, n0, a.N, kt * kGemmK, lb, wave, lane);
  };
  auto compute = [&](const uint8_t* la, const uint8_t* lb) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < kGemmK / 32; ++ks) {
      u32x4 fb[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        fb[nb] = *reinterpret_cast<const u32x4*>(lb + gemm_lds_offset(wn * 64 + nb * 16 + c16, ks * 4 + g));
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const u32x4 fa =
            *reinterpret_cast<const u32x4*>(la + gemm_lds_offset(wm * 128 + mb * 16 + c16, ks * 4 + g));
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma_bf16(fb[nb], fa, acc[mb][nb]);
      }
    }
  };

  load(0, sa0, sb0);
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {  // unrolled by two: each stage a fixed LDS object
    load(kt + 1, sa1, sb1);
    compute(sa0, sb0);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    if (kt + 2 < nk) load(kt + 2, sa0, sb0);
    compute(sa1, sb1);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
  }
  if (kt < nk) compute(sa0, sb0);

  // D = W-rows x A-rows^T per block: element i is output feature 16 nb + 4 g + i
  // (of the wave's 64) for token 16 mb + c16; four consecutive features per lane
  // are stored as one 8-byte bf16 group
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    const long long m = m0 + wm * 128 + mb * 16 + c16;
    if (m >= a.M) continue;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const long long n = n0 + wn * 64 + nb * 16 + 4 * g;
      uint16_t* dst = a.y + m * a.N + n;
      if (n + 3 < a.N) {
        const u32x2 v{pack_bf16x2(acc[mb][nb][0], acc[mb][nb][1]),
                      pack_bf16x2(acc[mb][nb][2], acc[mb][nb][3])};
        *reinterpret_cast<u32x2*>(dst) = v;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (n + i < a.N) dst[i] = f32_to_bf16(acc[mb][nb][i]);
      }
    }
  }
}

}  // namespace

hipError_t launch_lambda_proj(const LambdaProjArgs& a, hipStream_t stream) {
  const long long blocks = (a.N + kProjTokens - 1) / kProjTokens;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks), block(kProjWaves * kWave);
  switch (a.h / 16) {
    case 1: hipLaunchKernelGGL((lambda_proj_kernel<1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((lambda_proj_kernel<2>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((lambda_proj_kernel<3>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((lambda_proj_kernel<4>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_tn(const GemmArgs& a, hipStream_t stream) {
  const long long tiles = ((a.M + kGemmTile - 1) / kGemmTile) * ((a.N + kGemmTile - 1) / kGemmTile);
  if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(gemm_tn_kernel, dim3((unsigned)tiles), dim3(kGemmWaves * kWave), 0, stream, a);
  return hipGetLastError();
}

}  // namespace diffattn
