// bf16 MFMA GEMM for the ranker's projections: C = epi(A W^T) with A the
// packed activation rows [M, K] and W a weight matrix in nn.Linear layout
// [N, K].  Both operands are K-contiguous, so each 16-byte chunk of a row is
// exactly the 8 bf16 values one lane feeds to v_mfma_f32_32x32x16_bf16.
//
// Design (gfx950 / CDNA4):
//   * block tile BM x BN x 64, WM x WN waves, each wave owning a
//     (BM/WM) x (BN/WN) sub-tile of 32x32 MFMA blocks accumulated in fp32;
//   * operands staged global -> registers -> LDS, two LDS stages so the next
//     k-slab's global loads are in flight while the current one is multiplied;
//     one barrier per k-slab;
//   * LDS rows are 128 bytes (64 bf16); the 16-byte chunk index is XOR-swizzled
//     with (row >> 1) & 7 so the 16 lanes of a ds_read_b128 phase hit 64
//     distinct banks;
//   * the k loop order is fixed and there is no split-K, so every output row
//     is computed by the same instruction sequence whatever M is or where the
//     row sits: results are batch invariant;
//   * epilogues: bf16 store (QKV), fp32 residual add (O-proj, down-proj),
//     SwiGLU on interleaved gate/up column blocks (gate/up projection).
#include "launch.h"

namespace duolm {

namespace {

constexpr int BK = 64;

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(WM * WN * 64) void k_gemm(const uint16_t* __restrict__ A, int lda,
                                                      const uint16_t* __restrict__ W, int ldw,
                                                      void* __restrict__ Cv, int ldc,
                                                      const int32_t* __restrict__ dM, int N, int K) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / 32, NI = WTN / 32;
  constexpr int A_PER_T = BM * BK / 8 / NT;
  constexpr int B_PER_T = BN * BK / 8 / NT;
  static_assert(A_PER_T * NT * 8 == BM * BK && B_PER_T * NT * 8 == BN * BK, "tile/thread mismatch");
  static_assert(EPI != EPI_SWIGLU || NI % 2 == 0, "swiglu needs gate/up block pairs");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2][(BM + BN) * BK];

  const int M = *dM;
  const int n_tiles = N / BN;
  const int tile_n = blockIdx.x % n_tiles;
  const int tile_m = blockIdx.x / n_tiles;
  const int m0 = tile_m * BM, n0 = tile_n * BN;
  if (m0 >= M) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // global -> register staging
  uint4 ra[A_PER_T], rb[B_PER_T];
  const uint16_t* a_ptr[A_PER_T];
  const uint16_t* b_ptr[B_PER_T];
  int a_lds[A_PER_T], b_lds[B_PER_T];
#pragma unroll
  for (int i = 0; i < A_PER_T; ++i) {
    const int c = tid + i * NT;
    const int r = c >> 3, kc = c & 7;
    const int gr = min(m0 + r, M - 1);  // rows past M load a valid row; never stored
    a_ptr[i] = A + (size_t)gr * lda + kc * 8;
    a_lds[i] = r * BK + ((kc ^ swz(r)) << 3);
  }
#pragma unroll
  for (int i = 0; i < B_PER_T; ++i) {
    const int c = tid + i * NT;
    const int r = c >> 3, kc = c & 7;
    b_ptr[i] = W + (size_t)(n0 + r) * ldw + kc * 8;
    b_lds[i] = BM * BK + r * BK + ((kc ^ swz(r)) << 3);
  }

  // per-lane LDS fragment offsets (in elements) for k-step 0
  int a_frag[MI], b_frag[NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) a_frag[mi] = (wm * WTM + mi * 32 + (lane & 31)) * BK;
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) b_frag[ni] = BM * BK + (wn * WTN + ni * 32 + (lane & 31)) * BK;
  const int half = lane >> 5;

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  auto load_global = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_ptr[i] + kt * BK);
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) rb[i] = *reinterpret_cast<const uint4*>(b_ptr[i] + kt * BK);
  };
  auto store_lds = [&](int st) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) *reinterpret_cast<uint4*>(&smem[st][a_lds[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) *reinterpret_cast<uint4*>(&smem[st][b_lds[i]]) = rb[i];
  };

  const int KT = K / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < KT) load_global(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kc = ks * 2 + half;
      bf16x8_t af[MI], bfr[NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int r = wm * WTM + mi * 32 + (lane & 31);
        af[mi] = *reinterpret_cast<const bf16x8_t*>(&smem[st][a_frag[mi] + ((kc ^ swz(r)) << 3)]);
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int r = wn * WTN + ni * 32 + (lane & 31);
        bfr[ni] = *reinterpret_cast<const bf16x8_t*>(&smem[st][b_frag[ni] + ((kc ^ swz(r)) << 3)]);
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < KT) store_lds(st ^ 1);
    __syncthreads();
  }

  // epilogue: acc[mi][ni][r] = C[row][col], row = (r/4)*8 + half*4 + r%4, col = lane%32
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * WTM + mi * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
      if (row >= M) continue;
      if constexpr (EPI == EPI_BF16) {
        uint16_t* C = reinterpret_cast<uint16_t*>(Cv) + (size_t)row * ldc;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) C[n0 + wn * WTN + ni * 32 + (lane & 31)] = f32_to_bf16(acc[mi][ni][r]);
      } else if constexpr (EPI == EPI_RESID) {
        float* C = reinterpret_cast<float*>(Cv) + (size_t)row * ldc;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) C[n0 + wn * WTN + ni * 32 + (lane & 31)] += acc[mi][ni][r];
      } else {
        uint16_t* C = reinterpret_cast<uint16_t*>(Cv) + (size_t)row * ldc;
#pragma unroll
        for (int ni = 0; ni < NI; ni += 2) {
          const float g = acc[mi][ni][r], u = acc[mi][ni + 1][r];
          const float h = g / (1.0f + __expf(-g)) * u;
          C[(n0 + wn * WTN + ni * 32) / 2 + (lane & 31)] = f32_to_bf16(h);
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
void launch_cfg(hipStream_t s, int epi, int cap_m, const uint16_t* A, int lda, const uint16_t* W, int ldw,
                void* C, int ldc, const int32_t* dM, int N, int K) {
  const int grid = ((cap_m + BM - 1) / BM) * (N / BN);
  const dim3 blk(WM * WN * 64);
  if (epi == EPI_BF16)
    hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, EPI_BF16>), dim3(grid), blk, 0, s, A, lda, W, ldw, C, ldc, dM, N, K);
  else if (epi == EPI_RESID)
    hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, EPI_RESID>), dim3(grid), blk, 0, s, A, lda, W, ldw, C, ldc, dM, N, K);
  else
    hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, EPI_SWIGLU>), dim3(grid), blk, 0, s, A, lda, W, ldw, C, ldc, dM, N, K);
}

}  // namespace

bool launch_gemm(hipStream_t s, int epi, int cap_m, const uint16_t* A, int lda, const uint16_t* W, int ldw,
                 void* C, int ldc, const int32_t* dM, int N, int K) {
  if (N % 64 != 0 || K % BK != 0 || N <= 0 || K <= 0) return false;
  if (cap_m <= 0) return true;
  // Tile choice: the largest tile that still gives at least one block per CU
  // (256 CUs); small problems fall back to 64-wide tiles.
  const long tiles256 = (long)((cap_m + 255) / 256) * (N % 256 == 0 ? N / 256 : 0);
  const long tiles128 = (long)((cap_m + 127) / 128) * (N % 128 == 0 ? N / 128 : 0);
  if (N % 256 == 0 && tiles256 >= 256)
    launch_cfg<256, 256, 2, 2>(s, epi, cap_m, A, lda, W, ldw, C, ldc, dM, N, K);
  else if (N % 128 == 0 && tiles128 >= 128)
    launch_cfg<128, 128, 2, 2>(s, epi, cap_m, A, lda, W, ldw, C, ldc, dM, N, K);
  else
    launch_cfg<64, 64, 1, 1>(s, epi, cap_m, A, lda, W, ldw, C, ldc, dM, N, K);
  return true;
}

}  // namespace duolm
