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
//     them; the self term is merged into the online softmax at the end.
//
// Orientation: each wave computes S^T = K Q^T for 32 query columns (a column
// is one (row, query head) pair of the KV head's group) with
// v_mfma_f32_32x32x16_bf16, so a lane owns one query and 32 of the 64 keys of
// a tile; then O^T = V^T P^T, so the softmax statistics of a query never
// leave its lane.  K tiles sit in LDS row-major with a 16-byte-chunk XOR
// swizzle; V tiles are stored transposed (dims x keys, padded rows).
#include "launch.h"

namespace duolm {

namespace {

constexpr int BKV = 64;        // keys per tile
constexpr int VT_LD = BKV + 4; // padded row of the transposed V tile (elements)

// One instantiation serves both row kinds (`branch` is a runtime flag), so a
// candidate row and a causal row run the very same instruction sequence.
template <int HD, int NW>
__global__ __launch_bounds__(NW * 64) void k_attn(const uint16_t* __restrict__ QKV, int ld,
                                                 uint16_t* __restrict__ O, int ldo, DevBatch b, int H,
                                                 int Hkv, float scale_log2, int branch) {
  const bool BRANCH = branch != 0;
  constexpr int NT = NW * 64;
  constexpr int NKS = HD / 16;  // k-steps of the QK^T product
  constexpr int NDB = HD / 32;  // 32-dim blocks of the output
  constexpr int CPR = HD / 8;   // 16-byte chunks per key row
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BKV * HD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[HD * VT_LD];

  const int n_items = BRANCH ? b.hdr->n_bitems : b.hdr->n_pitems;
  if ((int)blockIdx.x >= n_items) return;
  const WorkItem item = (BRANCH ? b.bitems : b.pitems)[blockIdx.x];
  const SeqDesc sd = b.seqs[item.seq];
  const int g = blockIdx.y;  // KV head
  const int G = H / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int qc = wave * 32 + (lane & 31);
  const int lrow = qc / G;
  const int hq = g * G + qc % G;
  const int rows_per_item = NW * 32 / G;

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
    qvalid = j < sd.K;
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
  // a wave whose 32 columns are all padding only helps stage tiles
  const bool wave_active = __any(qvalid);
  const size_t qrow = (size_t)(sd.row_off + qrel);
  const int kcol = H * HD + g * HD;
  const int vcol = H * HD + Hkv * HD + g * HD;

  bf16x8_t qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8_t*>(QKV + qrow * ld + hq * HD + ks * 16 + half * 8);

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  const uint16_t* seq_base = QKV + (size_t)sd.row_off * ld;

  for (int k0 = 0; k0 < kend; k0 += BKV) {
    __syncthreads();
    // K tile, row-major with swizzled chunks
    for (int c = tid; c < BKV * CPR; c += NT) {
      const int key = c / CPR, dc = c % CPR;
      const int kr = min(k0 + key, kend - 1);
      const uint4 v = *reinterpret_cast<const uint4*>(seq_base + (size_t)kr * ld + kcol + dc * 8);
      *reinterpret_cast<uint4*>(&Ks[key * HD + ((dc ^ (key % CPR)) << 3)]) = v;
    }
    // V tile, transposed: 4 keys x 8 dims per unit, written as 8 x (4 keys)
    for (int u = tid; u < (BKV / 4) * CPR; u += NT) {
      const int kq = u / CPR, dc = u % CPR;
      uint4 v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kr = min(k0 + kq * 4 + e, kend - 1);
        v[e] = *reinterpret_cast<const uint4*>(seq_base + (size_t)kr * ld + vcol + dc * 8);
      }
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int word = dd >> 1, sh = (dd & 1) * 16;
        auto pick = [&](const uint4& x) -> uint32_t {
          const uint32_t w = word == 0 ? x.x : word == 1 ? x.y : word == 2 ? x.z : x.w;
          return (w >> sh) & 0xffffu;
        };
        uint2 o;
        o.x = pick(v[0]) | (pick(v[1]) << 16);
        o.y = pick(v[2]) | (pick(v[3]) << 16);
        *reinterpret_cast<uint2*>(&Vt[(dc * 8 + dd) * VT_LD + kq * 4]) = o;
      }
    }
    __syncthreads();
    if (!wave_active) continue;

    // S^T for two 32-key blocks
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      const int key = kb * 32 + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int dc = ks * 2 + half;
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&Ks[key * HD + ((dc ^ (key % CPR)) << 3)]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
      }
    }
    // mask, scale (log2 domain), tile max
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = k0 + kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
        const float v = (kk <= klim && kk < kend) ? s[kb][r] * scale_log2 : -INFINITY;
        s[kb][r] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float mnew = fmaxf(m, tmax);
    const float msafe = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = exp2f(m - msafe);
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(s[kb][r] - msafe);
        s[kb][r] = p;
        psum += p;
      }
    lsum = __builtin_fmaf(lsum, alpha, psum);
    m = mnew;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

    // O^T += V^T P^T over 4 k-steps of 16 keys
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2) {
      const int kb = ks2 >> 1, rb = (ks2 & 1) * 8;
      bf16x8_t pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)s[kb][rb + e];
      const int key_lo = kb * 32 + (rb >> 2) * 8 + half * 4;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int dim = db * 32 + (lane & 31);
        const uint2 lo = *reinterpret_cast<const uint2*>(&Vt[dim * VT_LD + key_lo]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&Vt[dim * VT_LD + key_lo + 8]);
        const uint4 w = make_uint4(lo.x, lo.y, hi.x, hi.y);
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, w);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[db], 0, 0, 0);
      }
    }
  }

  if (wave_active) {
    // diagonal term: the row's own key and value
    const uint16_t* kself = QKV + qrow * ld + kcol;
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8_t kv = *reinterpret_cast<const bf16x8_t*>(kself + ks * 16 + half * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) part = __builtin_fmaf((float)qf[ks][e], (float)kv[e], part);
    }
    const float dot = part + __shfl_xor(part, 32, 64);
    const float sv = dot * scale_log2;
    const float mnew = fmaxf(m, sv);
    const float alpha = exp2f(m - mnew);
    const float ps = exp2f(sv - mnew);
    lsum = __builtin_fmaf(lsum, alpha, half == 0 ? ps : 0.f);
    m = mnew;
    const uint16_t* vself = QKV + qrow * ld + vcol;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const uint2 vv = *reinterpret_cast<const uint2*>(vself + db * 32 + i4 * 8 + half * 4);
        const float v4[4] = {bf16_to_f32(vv.x & 0xffffu), bf16_to_f32(vv.x >> 16), bf16_to_f32(vv.y & 0xffffu),
                             bf16_to_f32(vv.y >> 16)};
#pragma unroll
        for (int j = 0; j < 4; ++j) oacc[db][i4 * 4 + j] = __builtin_fmaf(ps, v4[j], oacc[db][i4 * 4 + j] * alpha);
      }
  }

  if (!qvalid) return;
  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  const float inv = 1.0f / ltot;
  uint16_t* orow = O + qrow * ldo + hq * HD;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      uint2 o;
      o.x = pack_bf16x2(oacc[db][i4 * 4 + 0] * inv, oacc[db][i4 * 4 + 1] * inv);
      o.y = pack_bf16x2(oacc[db][i4 * 4 + 2] * inv, oacc[db][i4 * 4 + 3] * inv);
      *reinterpret_cast<uint2*>(orow + db * 32 + i4 * 8 + half * 4) = o;
    }
}

constexpr int NW = 8;  // 256 query columns per workgroup

template <int HD>
void launch_hd(hipStream_t s, bool branch, int cap_items, const uint16_t* QKV, int ld, uint16_t* O, int ldo,
               DevBatch b, int H, int Hkv, float scale_log2) {
  const dim3 grid(cap_items, Hkv);
  hipLaunchKernelGGL((k_attn<HD, NW>), grid, dim3(NW * 64), 0, s, QKV, ld, O, ldo, b, H, Hkv, scale_log2,
                     branch ? 1 : 0);
}

}  // namespace

int attn_rows_per_item(bool, int group) { return NW * 32 / group; }

bool attn_supported(int hd) { return hd == 32 || hd == 64 || hd == 128; }

void launch_attn(hipStream_t s, bool branch, int hd, int cap_items, const uint16_t* QKV, int ld, uint16_t* O,
                 int ldo, DevBatch b, int H, int Hkv, float scale_log2) {
  if (cap_items <= 0) return;
  if (hd == 128) launch_hd<128>(s, branch, cap_items, QKV, ld, O, ldo, b, H, Hkv, scale_log2);
  else if (hd == 64) launch_hd<64>(s, branch, cap_items, QKV, ld, O, ldo, b, H, Hkv, scale_log2);
  else launch_hd<32>(s, branch, cap_items, QKV, ld, O, ldo, b, H, Hkv, scale_log2);
}

}  // namespace duolm
