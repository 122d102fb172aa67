// Attention of the MIS ranker forward on gfx950, flash-style with bf16 MFMA
// and fp32 online softmax, one kernel template for both row kinds:
//
//   prefix tiles (BRANCH = false): causal attention of prefix rows over the
//     prefix, per sequence -- the prefix is prefilled once per request;
//   branch tiles (BRANCH = true): every candidate row attends to the L prefix
//     keys plus its own key (the diagonal term), never to another candidate
//     (tree mask of "DuoLM: Fast and Effective Personalized Recommendation
//     with Language Models", 核心方法 and 方法步骤详情 step 4).  One workgroup
//     takes up to 128 candidates x all query heads of one KV head, so each
//     request's prefix K/V for that head streams from memory once for all of
//     them; the self term is merged into the online softmax at the end.  A
//     candidate spread over M rows (an item of M vectors, same page, 实验结果
//     FIR m = 8) is a causal branch: row i also merges rows 0..i-1 of its own
//     branch before its own key.
//
// Orientation: each wave computes S^T = K Q^T for 32 query columns (a column
// is one (row, query head) pair of the KV head's group) with
// v_mfma_f32_32x32x16_bf16, so a lane owns one query and 32 of the 64 keys of
// a tile; then O^T = V^T P^T, so the softmax statistics of a query never
// leave its lane.  K and V tiles go global -> LDS directly
// (global_load_lds_dwordx4, double-buffered: the next tile is in flight while
// the current one is multiplied).  Both sit row-major (key x dims) with an
// XOR swizzle of their 16-byte chunks; the V operand of O^T = V^T P^T, which
// needs 4 consecutive keys of one dim per lane, comes straight out of the
// row-major tile through the gfx950 LDS transpose read ds_read_b64_tr_b16.
#include "launch.h"

namespace duolm {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) uint16_t lds_u16_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// 16 bytes per lane, global -> LDS; lane i lands at lds + 16 i.  M0 holds the
// wave's LDS destination; one wait state separates the M0 write from the load
// that reads it.  Written as inline asm so that the compiler does not count
// it against the LDS reads (it would then make every fragment read wait for
// all LDS traffic); the kernel waits for it with s_waitcnt vmcnt before the
// barrier that publishes the tile.  The instruction has no register
// result (its data goes to LDS), so no register the compiler reallocates can
// be written by it while it is in flight; its address VGPRs and M0 are read
// when it issues, as with the builtin form of the same load.
__device__ __forceinline__ void load_lds16(const uint16_t* g, lds_u16_t* lds) {
  const uint32_t base = (uint32_t)(uintptr_t)lds;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(base) : "memory");
}
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Within each 16-lane group, lane i gets element i % 4 of the 8-byte reads of
// lanes 4j + i / 4 (j = 0..3): with lane i addressing row r0 + i / 4 at
// column c0 + 4 (i % 4) of a row-major 16-bit matrix, it receives column
// c0 + i of rows r0 .. r0 + 3.
__device__ __forceinline__ v4i16_t lds_read_tr16(const lds_u16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)p);
}

// One instantiation serves both row kinds, so a candidate row and a causal
// row run the very same instruction sequence.  A launch may carry both kinds,
// side by side on the chip (both are latency-bound, one workgroup per CU).
// The grid is one-dimensional and item-major: block b takes KV head b % Hkv
// of item b / Hkv, branch items [0, bcap) first, then the prefix items, each
// list longest first.  So all heads of the longest items go out first and
// the launch ends on short items (dispatching head by head had left the
// longest items' last heads for the end: branch launch 48.9 -> 41.7 us).
// V chunk swizzle: the four consecutive keys of a transpose read land in four
// different 16-chunk quarters of the bank space.
template <int CPR>
__device__ __forceinline__ int vswz_t(int key) {
  return ((key & 3) << 2) & (CPR - 1);
}

// v_exp_f32: 2^x, results below the normal range flush to zero (a softmax
// weight that small is dropped either way)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A column keeps exponentiating against a running maximum that may lag its
// true maximum by up to 2^TAU (so weights stay below 2^TAU, harmless in fp32
// and bf16), and rescales its sum and output only when a tile's maximum
// exceeds it by more than that.
constexpr float kLazyTau = 8.0f;

// BRANCH_ONLY: a launch of branch tiles alone (no prefix tiles), compiled as an
// instantiation of its own so that profiles tell it apart from the launches
// that carry prefix tiles; every row runs the same arithmetic in both.
template <int HD, int NW, int BKV, bool BRANCH_ONLY>
__global__ __launch_bounds__(NW * 64) void k_attn(const uint16_t* __restrict__ QKV, int ld,
                                                 uint16_t* __restrict__ O, int ldo, DevBatch b, int H,
                                                 int Hkv, float scale_log2, int bcap) {
  const int slot = (int)blockIdx.x / Hkv;
  const bool BRANCH = BRANCH_ONLY || slot < bcap;
  const int idx = BRANCH ? slot : slot - bcap;
  constexpr int NKS = HD / 16;         // k-steps of the QK^T product
  constexpr int NDB = HD / 32;         // 32-dim blocks of the output
  constexpr int CPR = HD / 8;          // 16-byte chunks per key row / per query column
  constexpr int NC = NW * 32;          // query columns per workgroup
  constexpr int TILE = BKV * HD;       // elements of one K or V tile
  constexpr int KB = BKV / 32;         // 32-key blocks per tile
  static_assert(BKV == 32 || BKV == 64, "key tile");
  static_assert(kPageRows % BKV == 0, "a key tile lies in one session page");
  constexpr int QCH = NC * CPR;        // 16-byte chunks of the query / output block
  static_assert(QCH % (64 * NW) == 0, "staging layout");
  auto vswz = [](int key) { return vswz_t<CPR>(key); };
  auto cswz = [](int c) { return c & (CPR - 1); };  // chunk swizzle of a query column / own-key row
  // LDS: K and V tiles per pipeline stage, and the own-key block, which holds
  // the rows' own K and V and finally stages the output.  Each stage is an
  // array of its own, so the compiler can see that reads of one stage never
  // touch the global->LDS copies in flight into the other (one array indexed
  // by a runtime stage made it wait for those copies before every V read).
  __shared__ __attribute__((aligned(1024))) uint16_t sK0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sK1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sV0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sV1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t Own[NC * HD];

  // the item and the item count load together (the grid never exceeds the
  // item buffer, so the read is in bounds even for surplus blocks; testing
  // one of its fields in the exit condition keeps its load above the branch)
  const WorkItem item = (BRANCH ? b.bitems : b.pitems)[idx];
  const int n_items = BRANCH ? b.hdr->n_bitems : b.hdr->n_pitems;
  if (idx >= n_items || item.L < 1) return;
  struct {
    int row_off, L, K;
  } const sd = {item.row_off, item.L, item.K};
  const int g = (int)blockIdx.x % Hkv;  // KV head
  const int G = H / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qc = wave * 32 + (lane & 31);
  const int lrow = qc / G;
  const int rows_per_item = NC / G;
  // Branch tiles hold whole candidate branches of M rows (row i of a branch
  // sees the prefix and rows 0..i of its own branch).
  const int M = BRANCH ? item.M : 1;
  const int rows_used = rows_per_item / M * M;
  // the item's query rows, relative to the sequence start, and how many exist
  const int item_row0 = BRANCH ? sd.L + item.r0 : item.r0;
  const int item_nrows = min(rows_used, (BRANCH ? sd.K : sd.L) - item.r0);

  // Every query row sees a run of earlier keys plus its own key.  The earlier
  // keys stream through LDS in 64-key tiles; the row's own (diagonal) key is
  // merged into the online softmax after them.  A causal row r and a
  // candidate at logical position L therefore reduce over their keys in the
  // same order, so a candidate scored by MIS and the last row of the same
  // candidate's independent causal sequence get bit-identical attention.
  int qrel;     // query row relative to the sequence start
  bool qvalid;
  int klim;     // last streamed key this query may see (inclusive)
  int kend;     // keys [0, kend) are streamed
  if (BRANCH) {
    const int j = item.r0 + lrow;
    qvalid = lrow < item_nrows;
    qrel = sd.L + min(j, sd.K - 1);
    klim = sd.L - 1;
    kend = sd.L;
  } else {
    const int r = item.r0 + lrow;
    qvalid = r < sd.L;
    qrel = min(r, sd.L - 1);
    klim = qrel - 1;
    kend = min(item.r0 + rows_per_item - 1, sd.L - 1);
  }
  // Last key any valid column of this wave needs.  A tile past it is fully
  // masked for the whole wave: processing it would leave the running max,
  // sum and output unchanged, so the wave skips its MFMAs.  A wave whose 32
  // columns are all padding only helps stage tiles.
  int wave_klim = qvalid ? klim : -1;
  int wave_kmin = qvalid ? klim : INT32_MAX;  // tiles ending at or before it need no mask
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    wave_klim = max(wave_klim, __shfl_xor(wave_klim, o, 64));
    wave_kmin = min(wave_kmin, __shfl_xor(wave_kmin, o, 64));
  }
  const bool wave_active = __any(qvalid);
  const int kcol = H * HD + g * HD;
  const int vcol = H * HD + Hkv * HD + g * HD;
  // packed rows: query row i of the item (and its own K/V) at qrow0 + i, prefix
  // key k at koff + k (offsets are virtual, so only these sums are addresses)
  const int qrow0 = sd.row_off + item_row0;
  lds_u16_t* const ldsOwn = (lds_u16_t*)(lds_void_t*)Own;
  // stage ST's K and V tiles
  auto kt = [&](auto st) -> uint16_t* { if constexpr (decltype(st)::value == 0) return sK0; else return sK1; };
  auto vt = [&](auto st) -> uint16_t* { if constexpr (decltype(st)::value == 0) return sV0; else return sV1; };

  // Query fragments straight from memory into registers: lane (column qc,
  // half h) holds chunks 2 ks + h (ks = 0 .. NKS-1) of its query, the B
  // operand of S^T = K Q^T.  Columns past the item's last row load the last
  // row (valid memory, never stored).
  bf16x8_t qf[NKS];
  {
    const uint16_t* qsrc =
        QKV + (size_t)(qrow0 + min(lrow, item_nrows - 1)) * ld + (g * G + qc % G) * HD + half * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qsrc + ks * 16);
  }

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  // Tile staging: one global_load_lds_dwordx4 fills 1 KB = 1024 / (2 HD)
  // consecutive keys.  K chunk dc of key k sits at slot dc ^ (k % CPR), V chunk
  // dc at slot dc ^ vswz(k); each lane fetches the chunk that belongs at its
  // slot.  Keys past kend load key kend - 1 (valid memory, masked out).
  // A tile's keys are consecutive rows of one source: rows of the packed QKV
  // buffer, or, for a session sequence, rows of one KV page (a page holds
  // kPageRows keys and tiles start at multiples of BKV, so a tile never
  // straddles two pages).
  constexpr int KPI = 1024 / (2 * HD);        // keys per load instruction
  constexpr int NLI = BKV / KPI;              // instructions per tile and matrix
  constexpr int LPW = (2 * NLI + NW - 1) / NW;  // instructions per wave (K and V)
  // Per-lane parts of each load, fixed for the item: the key within the tile
  // and the element offset of its chunk from the tile's first key row.  A
  // full tile then adds one wave-uniform row offset; only a tile that runs
  // past kend clamps its keys.
  const size_t key_stride = item.pt >= 0 ? (size_t)Hkv * HD : (size_t)ld;
  int k_in[LPW];
  size_t l_off[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int ins = wave + j * NW;  // wave-uniform
    const bool isv = ins >= NLI;
    const int key = (isv ? ins - NLI : ins) * KPI + lane / CPR;
    const int slot = lane % CPR;
    const int dc = slot ^ (isv ? vswz(key) : key % CPR);
    k_in[j] = key;
    l_off[j] = (size_t)key * key_stride +
               (item.pt >= 0 ? (size_t)(isv ? kPageRows * Hkv * HD : 0) + g * HD : (size_t)(isv ? vcol : kcol)) +
               dc * 8;
  }
  auto issue = [&](int k0, auto st) {
    lds_u16_t* const dK = (lds_u16_t*)(lds_void_t*)kt(st);
    lds_u16_t* const dV = (lds_u16_t*)(lds_void_t*)vt(st);
    const uint16_t* tbase;  // the tile's first key row
    if (item.pt >= 0) {
      const int pg = b.pages[item.pt + k0 / kPageRows];  // uniform over the tile
      tbase = b.kv + (int64_t)pg * b.page_stride + (size_t)(k0 % kPageRows) * (Hkv * HD);
    } else {
      tbase = QKV + (size_t)(item.koff + k0) * ld;
    }
    const bool full = k0 + BKV <= kend;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int ins = wave + j * NW;  // wave-uniform
      if (ins < 2 * NLI) {
        const bool isv = ins >= NLI;
        const uint16_t* src = tbase + l_off[j];
        if (!full) src += (ptrdiff_t)(min(k0 + k_in[j], kend - 1) - (k0 + k_in[j])) * (ptrdiff_t)key_stride;
        lds_u16_t* dst = (isv ? dV : dK) + (isv ? ins - NLI : ins) * KPI * HD;
        load_lds16(src, dst);
      }
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;

  // The rows' own K and V into the own-key block: own-K row r at [r HD],
  // own-V row r at [(rows_per_item + r) HD], chunk k at slot k ^ (r % CPR).
  auto issue_own = [&]() {
    const int sin = QCH / (64 * G);  // load instructions per matrix
    for (int ins = wave; ins < 2 * sin; ins += NW) {
      const bool isv = ins >= sin;
      const int c = (isv ? ins - sin : ins) * 64 + lane;
      const int r = c / CPR, slot = c % CPR;
      const int lr = min(r, item_nrows - 1);
      const uint16_t* src = QKV + (size_t)(qrow0 + lr) * ld + (isv ? vcol : kcol) + ((slot ^ cswz(r)) << 3);
      load_lds16(src, ldsOwn + (isv ? rows_per_item * HD : 0) + (c - lane) * 8);
    }
  };

  // What the first tile needs goes out at once: the query fragments (above)
  // and the first key tile.  The rows' own K and V are needed only by the
  // merge after the last tile, so they load under the last tile (with no
  // next tile to fetch there, they share the load path with nothing); an item
  // with no streamed keys loads them here.  (Loading them here with the first
  // tile held up its start: branch tiles 40.8 -> 40.1 us per launch with
  // them under the last tile, and 39.0 -> 37.7 us under the first, same
  // scores.)
  const int ntiles = (kend + BKV - 1) / BKV;
  if (ntiles > 0) issue(0, S0{});
  if (ntiles == 0) issue_own();
  wait_loads();
  __syncthreads();
  // Every load has landed (above); telling the compiler that the query
  // fragments are consumed here keeps its own wait for them (which would
  // count the key-tile loads in flight) out of the tile loop.
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) asm volatile("" ::"v"(qf[ks]));

  auto tile = [&](int t, auto st) {
    constexpr int ST = decltype(st)::value;
    const int k0 = t * BKV;
    // the next tile's K and V go out first: the other stage was released at
    // the last barrier, so the loads have the whole tile to land
    if (t + 1 < ntiles) issue(k0 + BKV, std::integral_constant<int, ST ^ 1>{});
    if (t + 1 == ntiles) issue_own();  // lands before the wait at this tile's end
    const uint16_t* const Kt = kt(st);
    const lds_u16_t* const vb = (const lds_u16_t*)(lds_void_t*)vt(st);
    const bool busy = wave_active && k0 <= wave_klim;
    f32x16_t s[KB];
    if (busy) {
    // S^T for the tile's 32-key blocks, their accumulation chains interleaved
    // and each k-step's key fragments read one step ahead
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
    auto kfrag = [&](int kb, int ks) {
      const int key = kb * 32 + (lane & 31);
      const int dc = ks * 2 + half;
      return *reinterpret_cast<const bf16x8_t*>(&Kt[key * HD + ((dc ^ (key % CPR)) << 3)]);
    };
    bf16x8_t a[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) a[kb] = kfrag(kb, 0);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8_t n[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) n[kb] = ks + 1 < NKS ? kfrag(kb, ks + 1) : a[kb];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb], qf[ks], s[kb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);  // the reads stay one k-step ahead of their MFMAs
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) a[kb] = n[kb];
    }
    }  // QK of this tile
    if (busy) {
    // tile max of the raw scores (masked keys -> -inf); the mask is only
    // evaluated on tiles that reach past some column's last visible key
    float tmax = -INFINITY;
    if (k0 + BKV - 1 <= wave_kmin) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[kb][r]);
    } else {
      // key k0 + kb*32 + (r/4)*8 + half*4 + r%4 is visible when it is at or
      // below klim (for every row kind klim < kend): one compare of the
      // register's constant offset against the lane's bound
      const int lim = klim - k0 - half * 4;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float v = (kb * 32 + (r >> 2) * 8 + (r & 3)) <= lim ? s[kb][r] : -INFINITY;
          s[kb][r] = v;
          tmax = fmaxf(tmax, v);
        }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    // running max in the log2 domain: scores scaled by log2(e)/sqrt(hd)
    const float tl = tmax * scale_log2;
    const bool grow = tl > m + kLazyTau;  // false for a fully masked tile
    if (__any(grow)) {                     // other columns multiply by exactly 1
      const float mnew = grow ? tl : m;
      const float alpha = grow ? fast_exp2(m - mnew) : 1.0f;
      lsum *= alpha;
      m = mnew;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    const float msafe = m == -INFINITY ? 0.f : m;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[kb][r], scale_log2, -msafe));
        s[kb][r] = p;
        psum += p;
      }
    lsum += psum;

    // O^T += V^T P^T over the tile's k-steps of 16 keys
#pragma unroll
    for (int ks2 = 0; ks2 < BKV / 16; ++ks2) {
      const int kb = ks2 >> 1, rb = (ks2 & 1) * 8;
      bf16x8_t pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)s[kb][rb + e];
      const int key_lo = kb * 32 + (rb >> 2) * 8 + half * 4;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        // lanes of a 16-group: dims d0 .. d0 + 15 of keys key_lo .. key_lo + 3
        // (and + 8 .. + 11); lane i addresses key (i / 4), dims 4 (i % 4) ..
        const int d0 = db * 32 + ((lane >> 4) & 1) * 16;
        const int kx = key_lo + ((lane & 15) >> 2);
        const int dx = d0 + 4 * (lane & 3);
        const v4i16_t lo = lds_read_tr16(vb + kx * HD + (((dx >> 3) ^ vswz(kx)) << 3) + (dx & 7));
        const v4i16_t hi = lds_read_tr16(vb + (kx + 8) * HD + (((dx >> 3) ^ vswz(kx + 8)) << 3) + (dx & 7));
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[db], 0, 0, 0);
      }
    }
    }  // wave computes this tile
    wait_loads();
    __syncthreads();
  };
  for (int t = 0; t < ntiles; t += 2) {
    tile(t, S0{});
    if (t + 1 < ntiles) tile(t + 1, S1{});
  }
  // (every load has landed and been published: at the start, or at the end
  // of the last tile)

  if (wave_active) {
    // The row's own key and, in a candidate branch, the earlier rows of its
    // branch: local rows lrow - i .. lrow of the block (i = the row's index
    // in its branch; tiles start at branch boundaries), merged in order, the
    // row's own key last.  Every lane runs the branch's M steps; a step past
    // the row's own key adds a zero weight, leaving the sums unchanged.
    const int nmerge = BRANCH ? lrow % M + 1 : 1;
    for (int e = 0; e < M; ++e) {
      const bool act = e < nmerge;
      const int kr = act ? lrow - nmerge + 1 + e : lrow;
      const uint16_t* kself = Own + kr * HD;
      // q . k over the lane's half of the dims, two products per instruction
      // (v_dot2c_f32_bf16: bf16 products are exact in fp32)
      float part = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8_t kv = *reinterpret_cast<const bf16x8_t*>(kself + (((ks * 2 + half) ^ cswz(kr)) << 3));
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const bf16x2_t qa = {qf[ks][2 * e2], qf[ks][2 * e2 + 1]};
          const bf16x2_t kb2 = {kv[2 * e2], kv[2 * e2 + 1]};
          part = __builtin_amdgcn_fdot2_f32_bf16(qa, kb2, part, false);
        }
      }
      const float dot = part + __shfl_xor(part, 32, 64);
      const float sv = dot * scale_log2;
      const bool grow = act && sv > m + kLazyTau;
      if (__any(grow)) {
        const float mnew = grow ? sv : m;
        const float alpha = grow ? fast_exp2(m - mnew) : 1.0f;
        lsum *= alpha;
        m = mnew;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }
      const float ps = act ? fast_exp2(sv - m) : 0.f;
      lsum += half == 0 ? ps : 0.f;
      const uint16_t* vself = Own + (rows_per_item + kr) * HD;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const uint2 vv = *reinterpret_cast<const uint2*>(vself + (((db * 4 + i4) ^ cswz(kr)) << 3) + half * 4);
          const float v4[4] = {bf16_to_f32(vv.x & 0xffffu), bf16_to_f32(vv.x >> 16), bf16_to_f32(vv.y & 0xffffu),
                               bf16_to_f32(vv.y >> 16)};
#pragma unroll
          for (int j = 0; j < 4; ++j) oacc[db][i4 * 4 + j] = __builtin_fmaf(ps, v4[j], oacc[db][i4 * 4 + j]);
        }
    }
  }
  __syncthreads();  // every wave is done with the own K and V in the own-key block
  if (wave_active) {
    // normalised output of this column into the own-key block, column layout
    // with its chunk swizzle
    if (qvalid) {
      const float ltot = lsum + __shfl_xor(lsum, 32, 64);
      const float inv = 1.0f / ltot;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          uint2 o;
          o.x = pack_bf16x2(oacc[db][i4 * 4 + 0] * inv, oacc[db][i4 * 4 + 1] * inv);
          o.y = pack_bf16x2(oacc[db][i4 * 4 + 2] * inv, oacc[db][i4 * 4 + 3] * inv);
          *reinterpret_cast<uint2*>(&Own[qc * HD + (((db * 4 + i4) ^ cswz(qc)) << 3) + half * 4]) = o;
        }
    }
  }
  __syncthreads();
  // rows of the item: G heads x HD contiguous per row, 16 bytes per lane
  uint16_t* const obase = O + (size_t)qrow0 * ldo + g * G * HD;
#pragma unroll
  for (int j = 0; j < QCH / (64 * NW); ++j) {
    const int c = (wave + j * NW) * 64 + lane;
    const int col = c / CPR, slot = c % CPR;
    const int lr = col / G;
    if (lr < item_nrows) {
      const uint4 v = *reinterpret_cast<const uint4*>(&Own[c * 8]);
      *reinterpret_cast<uint4*>(obase + (size_t)lr * ldo + (col % G) * HD + ((slot ^ cswz(col)) << 3)) = v;
    }
  }
}

constexpr int NW = 8;    // query columns per workgroup = 32 NW
constexpr int BKV = 64;  // keys per streamed tile

template <int HD>
void launch_hd(hipStream_t s, int cap_p, int cap_b, const uint16_t* QKV, int ld, uint16_t* O, int ldo,
               DevBatch b, int H, int Hkv, float scale_log2) {
  const dim3 grid((cap_p + cap_b) * Hkv);
  if (cap_p == 0)
    hipLaunchKernelGGL((k_attn<HD, NW, BKV, true>), grid, dim3(NW * 64), 0, s, QKV, ld, O, ldo, b, H, Hkv,
                       scale_log2, cap_b);
  else
    hipLaunchKernelGGL((k_attn<HD, NW, BKV, false>), grid, dim3(NW * 64), 0, s, QKV, ld, O, ldo, b, H, Hkv,
                       scale_log2, cap_b);
}

}  // namespace

int attn_rows_per_item(bool, int group) { return NW * 32 / group; }

bool attn_supported(int hd) { return hd == 32 || hd == 64 || hd == 128; }

void launch_attn(hipStream_t s, int hd, int cap_p, int cap_b, const uint16_t* QKV, int ld, uint16_t* O, int ldo,
                 DevBatch b, int H, int Hkv, float scale_log2) {
  if (cap_p + cap_b <= 0) return;
  if (hd == 128) launch_hd<128>(s, cap_p, cap_b, QKV, ld, O, ldo, b, H, Hkv, scale_log2);
  else if (hd == 64) launch_hd<64>(s, cap_p, cap_b, QKV, ld, O, ldo, b, H, Hkv, scale_log2);
  else launch_hd<32>(s, cap_p, cap_b, QKV, ld, O, ldo, b, H, Hkv, scale_log2);
}

}  // namespace duolm
