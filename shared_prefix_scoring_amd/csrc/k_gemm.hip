// bf16 MFMA GEMM for the ranker's projections: C = epi(A W^T) with A the
// packed activation rows [M, K] and W a weight matrix in nn.Linear layout
// [N, K].  Both operands are K-contiguous, so each 16-byte chunk of a row is
// exactly the 8 bf16 values one lane feeds to v_mfma_f32_32x32x16_bf16.
//
// Design (gfx950 / CDNA4):
//   * block tile BM x BN x 64, WM x WN waves, each wave owning a
//     (BM/WM) x (BN/WN) sub-tile of 32x32 MFMA blocks accumulated in fp32;
//     the large shape is 256 x 256 with 8 waves (two per SIMD, 64 x 128
//     each), so one wave's LDS and barrier waits overlap the other's MFMAs;
//   * operands go global -> LDS directly with global_load_lds_dwordx4 (one
//     instruction fills 1 KB of LDS = 8 rows of 128 bytes, lane i writing
//     bytes [16i, 16i+16)); no staging registers, so the accumulators can
//     fill the AGPR file and the loads of k-slab kt+1 fly while slab kt is
//     multiplied out of the other LDS stage;
//   * LDS rows are 128 bytes (64 bf16); the 16-byte chunk index is XOR-swizzled
//     with (row ^ (row >> 3)) & 7 -- each lane fetches the global chunk that
//     belongs at its LDS slot -- so the 32 rows of a fragment read hit
//     distinct bank groups;
//   * fragments are double-buffered in registers: the ds_read_b128s of k-step
//     ks+1 are issued among the MFMAs of k-step ks, in a fixed instruction
//     order held by scheduling fences (see the slab below);
//   * the global->LDS loads are written as inline asm: while the compiler's
//     own form of this load is in flight, it turns every fragment wait into
//     a wait for all outstanding LDS traffic; with the loads out of its view
//     each k-step waits only for the fragments its first MFMAs need, and the
//     kernel waits for the loads itself (vmcnt) before the stage barrier;
//   * persistent: at most one workgroup per CU, each walking its tiles
//     round by round in an XCD-aware order (see the kernel); a tile's last
//     slab loads the next tile's first slab into the free stage, and that
//     load lands while the tile's epilogue runs (no relaunch, no exposed
//     first-slab latency);
//   * a launch with fewer tiles than CUs runs one tile per workgroup on a
//     deeper LDS ring (NS stages), its loads several slabs ahead;
//   * the k loop order is fixed and there is no split-K, so every output row
//     is computed by the same instruction sequence whatever M is or where the
//     row sits: results are batch invariant;
//   * epilogues: bf16 store (QKV), fp32 residual add (O-proj, down-proj),
//     SwiGLU on interleaved gate/up column blocks (gate/up projection).
#include <algorithm>
#include <type_traits>

#include "launch.h"

namespace duolm {

namespace {

constexpr int BK = 64;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) uint16_t lds_u16_t;

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// 16 bytes per lane, global -> LDS; lane i lands at lds + 16 i.  M0 holds the
// wave's LDS destination; one wait state separates the M0 write from the load
// that reads it.  Nothing is returned to registers: the caller waits with
// s_waitcnt vmcnt before the barrier that publishes the stage.  The instruction has no register
// result (its data goes to LDS), so no register the compiler reallocates can
// be written by it while it is in flight; its address VGPRs and M0 are read
// when it issues, as with the builtin form of the same load.
__device__ __forceinline__ void load_lds16(const uint16_t* g, lds_u16_t* lds) {
  const uint32_t base = (uint32_t)(uintptr_t)lds;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(base) : "memory");
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// wait until at most N of this wave's global->LDS loads are in flight (they
// complete in issue order)
template <int N>
__device__ __forceinline__ void wait_loads_but() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// NS: LDS stages.  NS = 2 is the persistent double-buffered loop; NS > 2 is
// for launches whose tiles fit one per CU (one tile per workgroup).
template <int BM, int BN, int WM, int WN, int EPI, int NS>
__global__ __launch_bounds__(WM * WN * 64) void k_gemm(const uint16_t* __restrict__ A, int lda,
                                                      const uint16_t* __restrict__ W, int ldw,
                                                      void* __restrict__ Cv, int ldc,
                                                      const int32_t* __restrict__ dM, int N, int K,
                                                      int xg) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / 32, NI = WTN / 32;
  constexpr int GA = BM / 8 / NW, GB = BN / 8 / NW;  // 8-row groups each wave loads
  constexpr int STAGE = (BM + BN) * BK;               // elements per LDS stage
  static_assert(GA * NW * 8 == BM && GB * NW * 8 == BN, "tile/wave mismatch");
  static_assert(EPI != EPI_SWIGLU || NI % 2 == 0, "swiglu needs gate/up block pairs");

  static_assert(NS >= 2, "stages");
  __shared__ __attribute__((aligned(1024))) uint16_t smem[NS * STAGE];

  const int M = *dM;
  const int n_tiles = N / BN;
  const int nblk = __builtin_amdgcn_readfirstlane(gridDim.x);
  // Tile order.  Workgroups are dispatched to the 8 XCDs round-robin
  // (workgroup b on XCD b % 8), and each XCD has its own L2.  With xg > 0
  // the column tiles are split into xg groups; XCD x works only on group
  // x % xg, and takes the group's tiles (row-major) in runs of consecutive
  // tiles, so the workgroups of one XCD share their A row blocks and their
  // group's weight columns in that XCD's L2.  Round k hands out the group's
  // tiles [k stride, (k + 1) stride): a full round gives each of the group's
  // nx XCDs a run of `per` tiles (one per workgroup); a partial last round is
  // split into nx runs as equal as can be, so no XCD is left holding the
  // tail while another idles (a second launch beside this one waits for the
  // XCD its next workgroup is dispatched to).
  int grp = 0, q = 0, j = blockIdx.x, per = nblk, nx = 1, stride = nblk, ncol = n_tiles;
  if (xg > 0 && nblk % 8 == 0 && n_tiles % xg == 0 && 8 % xg == 0) {
    const int x = blockIdx.x % 8;
    per = nblk / 8;
    nx = 8 / xg;
    grp = x % xg;
    q = x / xg;
    j = blockIdx.x / 8;
    stride = nblk / xg;
    ncol = n_tiles / xg;
  }
  const int total = (M + BM - 1) / BM * ncol;  // tiles of this workgroup's group
  // index (row-major within the group) of this workgroup's tile in round k, or -1
  auto tile_at = [&](int k) -> int {
    const int base = k * stride;
    if (base + stride <= total) return base + q * per + j;
    const int r = total - base;
    if (r <= 0) return -1;
    const int chunk = (r + nx - 1) / nx;
    return j < chunk && q * chunk + j < r ? base + q * chunk + j : -1;
  };
  const int first = tile_at(0);
  if (first < 0) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5;
  const int KT = K / BK;

  // Load cursor: tile lt, slab lk go out next.  Per-lane source of this
  // wave's row groups: row g*8 + lane/8, the chunk whose swizzled slot is lane%8
  const uint16_t* pa[GA];
  const uint16_t* pb[GB];
  int lt = first, lround = 0, lk = 0;
  auto aim = [&](int tt) {
    const int m0 = tt / ncol * BM, n0 = (grp * ncol + tt % ncol) * BN;
#pragma unroll
    for (int j = 0; j < GA; ++j) {
      const int r = (wave + NW * j) * 8 + (lane >> 3);
      const int kc = (lane & 7) ^ swz(r);
      pa[j] = A + (size_t)min(m0 + r, M - 1) * lda + kc * 8;  // rows past M load a valid row, never stored
    }
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      const int r = (wave + NW * j) * 8 + (lane >> 3);
      const int kc = (lane & 7) ^ swz(r);
      pb[j] = W + (size_t)(n0 + r) * ldw + kc * 8;
    }
  };
  aim(lt);
  auto advance = [&]() {
    if (++lk == KT) {
      lk = 0;
      lt = tile_at(++lround);
      if (lt >= 0) aim(lt);
    }
  };
  lds_u16_t* lds = (lds_u16_t*)(lds_void_t*)smem;


  // fragment rows and their swizzles
  int a_row[MI], a_sw[MI], b_row[NI], b_sw[NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int r = wm * WTM + mi * 32 + (lane & 31);
    a_row[mi] = r * BK;
    a_sw[mi] = swz(r);
  }
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    const int r = wn * WTN + ni * 32 + (lane & 31);
    b_row[ni] = BM * BK + r * BK;
    b_sw[ni] = swz(r);
  }

  bf16x8_t fa[2][MI], fb[2][NI];

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;


  constexpr int NM = MI * NI;          // MFMAs per k-step
  constexpr int NR = MI + NI;          // fragment reads per k-step
  constexpr int NG = GA + GB;          // global->LDS loads per slab
  // fragment reads in the order the MFMAs first use them: a[0], b[0..NI-1], a[1..MI-1]
  auto read_one = [&](int j, int st, int ks, int buf) {
    const int kc = ks * 2 + half;
    if (j == 0) {
      fa[buf][0] = *reinterpret_cast<const bf16x8_t*>(&smem[st * STAGE + a_row[0] + ((kc ^ a_sw[0]) << 3)]);
    } else if (j <= NI) {
      const int ni = j - 1;
      fb[buf][ni] = *reinterpret_cast<const bf16x8_t*>(&smem[st * STAGE + b_row[ni] + ((kc ^ b_sw[ni]) << 3)]);
    } else {
      const int mi = j - NI;
      fa[buf][mi] = *reinterpret_cast<const bf16x8_t*>(&smem[st * STAGE + a_row[mi] + ((kc ^ a_sw[mi]) << 3)]);
    }
  };
  auto issue_one = [&](int g, int st) {
    if (g < GA)
      load_lds16(pa[g] + lk * BK, lds + st * STAGE + (wave + NW * g) * 8 * BK);
    else
      load_lds16(pb[g - GA] + lk * BK, lds + st * STAGE + BM * BK + (wave + NW * (g - GA)) * 8 * BK);
  };
  auto mfma_one = [&](int buf, int i) {
    acc[i / NI][i % NI] =
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i / NI], fb[buf][i % NI], acc[i / NI][i % NI], 0, 0, 0);
  };
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  // One k-slab, in a fixed instruction order (scheduling fences between the
  // groups): k-step 0 interleaves its MFMAs with the next slab's global->LDS
  // loads and the fragment reads of k-step 1; k-steps 1 and 2 with the reads
  // of the step after; k-step 3 runs half its MFMAs, waits for the next slab
  // and meets the other waves at the barrier, then reads the next slab's
  // first fragments under the other half.
  // epilogue of the tile at (m0, n0): acc[mi][ni][r] = C[row][col],
  // row = (r/4)*8 + half*4 + r%4, col = lane%32
  auto epilogue = [&](int m0, int n0) {
    if constexpr (EPI == EPI_RESID) {
      // residual add, software-pipelined over groups of GR of a lane's rows:
      // the loads of group j + 1 are in flight while group j is added and
      // stored, so the epilogue pays about one memory latency in all rather
      // than one per group (rows past M read row M - 1 and are not stored)
      float* C = reinterpret_cast<float*>(Cv);
      constexpr int GR = NI >= 4 ? 4 : 8;  // rows per group: GR x NI loads in flight per buffer
      constexpr int NGR = MI * (16 / GR);
      float xv[2][GR][NI];
      auto row_of = [&](int j, int r) {
        return m0 + wm * WTM + (j / (16 / GR)) * 32 + (((j % (16 / GR)) * GR + r) >> 2) * 8 + half * 4 + (r & 3);
      };
      auto load_group = [&](int j, int buf) {
#pragma unroll
        for (int r = 0; r < GR; ++r) {
          const int row = min(row_of(j, r), M - 1);
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            xv[buf][r][ni] = C[(size_t)row * ldc + n0 + wn * WTN + ni * 32 + (lane & 31)];
        }
      };
      load_group(0, 0);
#pragma unroll
      for (int j = 0; j < NGR; ++j) {
        if (j + 1 < NGR) load_group(j + 1, (j + 1) & 1);
        const int mi = j / (16 / GR), r0 = (j % (16 / GR)) * GR;
#pragma unroll
        for (int r = 0; r < GR; ++r) {
          const int row = row_of(j, r);
          if (row < M) {
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
              C[(size_t)row * ldc + n0 + wn * WTN + ni * 32 + (lane & 31)] = xv[j & 1][r][ni] + acc[mi][ni][r0 + r];
          }
        }
      }
    } else {
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
          } else {
            uint16_t* C = reinterpret_cast<uint16_t*>(Cv) + (size_t)row * ldc;
#pragma unroll
            for (int ni = 0; ni < NI; ni += 2) {
              const float g = acc[mi][ni][r], u = acc[mi][ni + 1][r];
              // silu(g) u with the hardware reciprocal (about 1 ulp; the result
              // is rounded to bf16)
              const float h = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
              C[(n0 + wn * WTN + ni * 32) / 2 + (lane & 31)] = f32_to_bf16(h);
            }
          }
        }
      }
    }
  };

  if constexpr (NS > 2) {
    // One tile per workgroup, for launches whose tiles fit one per CU: an
    // NS-stage LDS ring whose loads run NS - 1 slabs ahead of the MFMAs, so
    // each slab's memory latency is hidden behind the slabs before it (with
    // two stages a small launch waits about one latency on every slab).  The
    // arithmetic is the two-stage loop's: the same k-steps in the same order.
    static_assert((NS - 2) * NG <= 63, "loads in flight");
    const int m0 = first / ncol * BM, n0 = (grp * ncol + first % ncol) * BN;
    for (int sl = 0; sl < NS - 1 && sl < KT; ++sl) {
      lk = sl;
#pragma unroll
      for (int g = 0; g < NG; ++g) issue_one(g, sl);
    }
    for (int kt = 0; kt < KT; ++kt) {
      // slab kt has landed (the loads of up to NS - 2 later slabs may fly),
      // and every wave is done with slab kt - 1, whose stage is refilled next
      if (kt + NS - 2 < KT)
        wait_loads_but<(NS - 2) * NG>();
      else
        wait_loads();
      __syncthreads();
      if (kt + NS - 1 < KT) {
        lk = kt + NS - 1;
        const int sn = lk % NS;
#pragma unroll
        for (int g = 0; g < NG; ++g) issue_one(g, sn);
      }
      const int st = kt % NS;
#pragma unroll
      for (int r = 0; r < NR; ++r) read_one(r, st, 0, 0);
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          mfma_one(ks & 1, i);
          if (ks + 1 < BK / 16) {
#pragma unroll
            for (int r = i * NR / NM; r < (i + 1) * NR / NM; ++r) read_one(r, st, ks + 1, (ks + 1) & 1);
          }
          fence();
        }
      }
    }
    epilogue(m0, n0);
  } else {
    // The last slab of a tile neither waits nor reads ahead: the next tile's
    // first slab (always issued; past the block's last tile it reloads a slab
    // of that tile into the free stage) lands under the epilogue.
    auto slab = [&](int st, auto is_last) {
      constexpr bool last = decltype(is_last)::value;
#pragma unroll
      for (int ks = 0; ks < 3; ++ks) {
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          mfma_one(ks & 1, i);
          if (ks == 0) {
#pragma unroll
            for (int g = i * NG / NM; g < (i + 1) * NG / NM; ++g) issue_one(g, st ^ 1);
          }
#pragma unroll
          for (int j = i * NR / NM; j < (i + 1) * NR / NM; ++j) read_one(j, st, ks + 1, (ks + 1) & 1);
          fence();
        }
        if (ks == 0) advance();
      }
#pragma unroll
      for (int i = 0; i < NM / 2; ++i) {
        mfma_one(1, i);
        fence();
      }
      if constexpr (!last) {
        wait_loads();
        __syncthreads();
      }
      fence();
#pragma unroll
      for (int i = NM / 2; i < NM; ++i) {
        mfma_one(1, i);
        if constexpr (!last) {
          const int i2 = i - NM / 2;
#pragma unroll
          for (int j = i2 * NR / (NM / 2); j < (i2 + 1) * NR / (NM / 2); ++j) read_one(j, st ^ 1, 0, 0);
        }
        fence();
      }
    };

#pragma unroll
    for (int g = 0; g < NG; ++g) issue_one(g, 0);
    advance();
    wait_loads();
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NR; ++j) read_one(j, 0, 0, 0);
    int st = 0;
    for (int ct = first, cround = 0;;) {
      for (int kt = 0; kt + 1 < KT; ++kt) {
        slab(st, std::false_type{});
        st ^= 1;
      }
      slab(st, std::true_type{});
      st ^= 1;
      epilogue(ct / ncol * BM, (grp * ncol + ct % ncol) * BN);
      ct = tile_at(++cround);
      if (ct < 0) break;
      // the next tile's first slab went out under this tile's last slab
      wait_loads();
      __syncthreads();
#pragma unroll
      for (int j = 0; j < NR; ++j) read_one(j, st, 0, 0);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
    }
    wait_loads();  // no load into LDS outlives the workgroup
  }
}

int cu_count() {
  static const int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    return v;
  }();
  return n;
}

template <int BM, int BN, int WM, int WN, int NS = 2>
void launch_cfg(hipStream_t s, int epi, int cap_m, const uint16_t* A, int lda, const uint16_t* W, int ldw,
                void* C, int ldc, const int32_t* dM, int N, int K) {
  // Two stages: persistent workgroups for the large tiles, whose LDS stages
  // (112-128 KB) allow one workgroup per CU: one per tile up to one per CU (a
  // two-lane split still gives each launch the whole chip: capping it at its
  // share of the CUs measured 6% slower per call).  Smaller tiles fit several
  // workgroups per CU, so they get one workgroup per tile.  Deeper rings:
  // one workgroup per tile.
  const int tiles = ((cap_m + BM - 1) / BM) * (N / BN);
  const int grid = NS == 2 && 2 * (BM + BN) * BK * 2 > 96 * 1024 ? std::min(tiles, cu_count()) : tiles;
  // Column groups for the XCD-aware tile order (see the kernel): the count
  // with the least estimated L2 fill traffic.  The activations are read once
  // per group (xg |A|); each of the 8 XCDs reads its group's share of the
  // weights once if that share fits its 4 MB L2, else once per round of
  // tiles.  At the 0.6B shape with 64 requests per call this picks 1 group
  // for the O and down projections (L2 fetch per launch 553 -> 275 MB), 2 for
  // QKV (405 -> 267 MB) and 4 for gate/up (473 -> 394 MB); per call 25.04 ->
  // 24.56 ms as one launch, 22.47 -> 22.31 ms as two lanes (A/B on one box,
  // scores bit-identical).
  constexpr double kL2Bytes = 4.0 * (1 << 20);
  const double a_bytes = 2.0 * cap_m * K, w_bytes = 2.0 * N * K;
  const int rounds = (tiles + grid - 1) / grid;
  int xg = 1;
  double best = -1.0;
  for (int g = 1; g <= 8 && (N / BN) % g == 0; g *= 2) {
    const double share = w_bytes / g;
    const double est = g * a_bytes + 8.0 * share * (share <= kL2Bytes ? 1 : rounds);
    if (best < 0 || est < best) {
      best = est;
      xg = g;
    }
  }
  const dim3 blk(WM * WN * 64);
  if (epi == EPI_BF16)
    hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, EPI_BF16, NS>), dim3(grid), blk, 0, s, A, lda, W, ldw, C,
                       ldc, dM, N, K, xg);
  else if (epi == EPI_RESID)
    hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, EPI_RESID, NS>), dim3(grid), blk, 0, s, A, lda, W, ldw, C,
                       ldc, dM, N, K, xg);
  else if constexpr ((BN / WN / 32) % 2 == 0)  // the chooser never asks others for SwiGLU
    hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, EPI_SWIGLU, NS>), dim3(grid), blk, 0, s, A, lda, W, ldw, C,
                       ldc, dM, N, K, xg);
}


}  // namespace

bool launch_gemm(hipStream_t s, int epi, int cap_m, const uint16_t* A, int lda, const uint16_t* W, int ldw,
                 void* C, int ldc, const int32_t* dM, int N, int K, int share) {
  if (N % 64 != 0 || K % BK != 0 || N <= 0 || K <= 0) return false;
  if (cap_m <= 0) return true;
  // Tile choice: the largest tile that still gives at least one block per CU;
  // small problems fall back to 64-wide tiles.  Every configuration reduces k
  // in the same order, so the choice never changes a result bit.  With one
  // tile per CU at a time, a launch takes (rounds of tiles) x (tile time); for
  // the residual projections (N = 1024: 336 tiles of 256 rows at T = 21.5k, a
  // two-round launch whose second round is a third full) 192-row tiles finish
  // in the same number of rounds with 3/4 of the work each, and are used
  // when they need fewer row-rounds -- for a launch that has the chip to
  // itself: beside the other half of a two-lane call, whose kernels fill the
  // last round's idle CUs, 256-row tiles measured faster (22.40 against
  // 22.59 ms per 64-request call).  (With the bf16 and SwiGLU epilogues the
  // 192-row tile measured slower.)
  // CUs this launch can expect: with `share` launches side by side (the
  // halves of a batch on two streams) a tile size that fills its share fills
  // the chip (measured: 24.45 against 25.15 ms per step for the 64-request batch)
  const int ncu = cu_count() / (share > 1 ? share : 1);
  const long nt = N % 256 == 0 ? N / 256 : 0;
  const long tiles256 = (long)((cap_m + 255) / 256) * nt;
  const long tiles128 = (long)((cap_m + 127) / 128) * (N % 128 == 0 ? N / 128 : 0);
  auto row_rounds = [&](int bm) { return ((((long)cap_m + bm - 1) / bm) * nt + ncu - 1) / ncu * bm; };
  if (nt && tiles256 >= ncu && epi == EPI_RESID && share <= 1 && row_rounds(192) < row_rounds(256))
    launch_cfg<192, 256, 2, 4>(s, epi, cap_m, A, lda, W, ldw, C, ldc, dM, N, K);
  else if (nt && tiles256 >= ncu)
    launch_cfg<256, 256, 4, 2>(s, epi, cap_m, A, lda, W, ldw, C, ldc, dM, N, K);
  else if (N % 128 == 0 && tiles128 >= ncu)
    launch_cfg<128, 128, 2, 2>(s, epi, cap_m, A, lda, W, ldw, C, ldc, dM, N, K);
  // Fewer tiles than CUs: one workgroup per CU, so a deep LDS ring fits
  // (4 x 32 KB or 8 x 16 KB) and hides the memory latency of each slab.
  // 64 x 64 tiles of four 32 x 32 waves double the workgroups of a narrow
  // projection; SwiGLU needs gate/up block pairs in a wave, so 128 x 128.
  else if (N % 128 == 0 && (tiles128 >= ncu / 4 || epi == EPI_SWIGLU))
    launch_cfg<128, 128, 2, 2, 4>(s, epi, cap_m, A, lda, W, ldw, C, ldc, dM, N, K);
  else if (N % 128 == 0)
    launch_cfg<64, 64, 2, 2, 8>(s, epi, cap_m, A, lda, W, ldw, C, ldc, dM, N, K);
  else
    launch_cfg<64, 64, 1, 1>(s, epi, cap_m, A, lda, W, ldw, C, ldc, dM, N, K);
  return true;
}

}  // namespace duolm
