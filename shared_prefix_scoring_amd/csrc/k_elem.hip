// Row-wise kernels of the ranker forward: VID-aware embedding gather,
// RMSNorm, per-head q/k RMSNorm + rotary embedding, and the score head.
// All are HBM-bound streaming kernels: one 64-lane wave per row (or per
// (row, head) group), 16-byte vector accesses, fp32 arithmetic.
#include "launch.h"

namespace duolm {

// ---------------------------------------------------------------------------
// Embedding gather over the extended vocabulary [0, V + N): ids below V read
// the bf16 token embedding, ids V + iota read row iota of the fp16 item table
// ("DuoLM: Fast and Effective Personalized Recommendation with Language
// Models", 方法步骤详情 step 3).  Ids V + N + j read row j of the call's
// inline item vectors (requests that ship vectors instead of ids).  All widen
// exactly to the fp32 residual stream.  Also writes each row's logical
// position: causal row rho -> rho, row i of every candidate branch -> L + i
// (same page, 核心方法 / step 4).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_embed(const int32_t* __restrict__ ids, DevBatch b,
                                               const uint16_t* __restrict__ E,
                                               const uint16_t* __restrict__ D,
                                               const uint16_t* __restrict__ Dinl, int V, int64_t n_vid,
                                               int d, float* __restrict__ X, int32_t* __restrict__ pos) {
  const int T = b.hdr->T;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= T) return;
  const int n = b.hdr->n_seq;
  const int seg = packed_segment(b.seq_row_off, 2 * n, row);  // branch segments first, then prefix ones
  const SeqDesc sd = b.seqs[seg < n ? seg : seg - n];
  const int rho = row - (seg < n ? sd.boff : sd.row_off);
  const int id = rho < sd.id_len ? ids[sd.id_off + rho] : ids[sd.cand_id_off + (rho - sd.id_len)];
  if (lane == 0) pos[row] = rho < sd.L ? rho : sd.L + (rho - sd.L) % sd.M;
  float* xr = X + (size_t)row * d;
  const int nchunk = d >> 3;  // 8 values per chunk
  if (id < 0 || (int64_t)id >= (int64_t)V + n_vid + b.hdr->n_inline) {
    if (lane == 0) atomicOr(b.err, 1);
    for (int c = lane; c < nchunk; c += 64) {
      reinterpret_cast<float4*>(xr + c * 8)[0] = make_float4(0.f, 0.f, 0.f, 0.f);
      reinterpret_cast<float4*>(xr + c * 8)[1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }
  const bool tok = id < V;
  const int64_t vrow = (int64_t)id - V;
  const uint16_t* src = tok ? E + (size_t)id * d
                            : (vrow < n_vid ? D + (size_t)vrow * d : Dinl + (size_t)(vrow - n_vid) * d);
  for (int c = lane; c < nchunk; c += 64) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + c * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t lo16 = (uint16_t)(w[e] & 0xffffu), hi16 = (uint16_t)(w[e] >> 16);
      f[2 * e] = tok ? bf16_to_f32(lo16) : f16_to_f32(lo16);
      f[2 * e + 1] = tok ? bf16_to_f32(hi16) : f16_to_f32(hi16);
    }
    reinterpret_cast<float4*>(xr + c * 8)[0] = make_float4(f[0], f[1], f[2], f[3]);
    reinterpret_cast<float4*>(xr + c * 8)[1] = make_float4(f[4], f[5], f[6], f[7]);
  }
}

void launch_embed(hipStream_t s, int cap_rows, const int32_t* ids, DevBatch b, const uint16_t* E,
                  const uint16_t* D, const uint16_t* Dinl, int V, int64_t n_vid, int d, float* X,
                  int32_t* pos) {
  if (cap_rows <= 0) return;
  hipLaunchKernelGGL(k_embed, dim3((cap_rows + 3) / 4), dim3(256), 0, s, ids, b, E, D, Dinl, V, n_vid, d, X,
                     pos);
}

// ---------------------------------------------------------------------------
// RMSNorm: y = x / sqrt(mean(x^2) + eps) * g, fp32 math, bf16 out.
// ---------------------------------------------------------------------------
// One wave per row.  The row stays in registers between the sum of squares
// and the scaling (NQ float4 per lane; NQ = 0 loops over the row instead).
template <int NQ>
__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ X, const float* __restrict__ g,
                                                 uint16_t* __restrict__ Y, const int32_t* __restrict__ n_rows,
                                                 int d, float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= *n_rows) return;
  const float4* xr = reinterpret_cast<const float4*>(X + (size_t)row * d);
  const float4* gr = reinterpret_cast<const float4*>(g);
  uint2* yr = reinterpret_cast<uint2*>(Y + (size_t)row * d);
  float ss = 0.f;
  if constexpr (NQ > 0) {
    float4 v[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) v[j] = xr[lane + 64 * j];
#pragma unroll
    for (int j = 0; j < NQ; ++j) ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const float4 gg = gr[lane + 64 * j];
      uint2 o;
      o.x = pack_bf16x2(v[j].x * inv * gg.x, v[j].y * inv * gg.y);
      o.y = pack_bf16x2(v[j].z * inv * gg.z, v[j].w * inv * gg.w);
      yr[lane + 64 * j] = o;
    }
  } else {
    const int nq = d >> 2;
    for (int c = lane; c < nq; c += 64) {
      const float4 v = xr[c];
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)d + eps);
    for (int c = lane; c < nq; c += 64) {
      const float4 v = xr[c];
      const float4 gg = gr[c];
      uint2 o;
      o.x = pack_bf16x2(v.x * inv * gg.x, v.y * inv * gg.y);
      o.y = pack_bf16x2(v.z * inv * gg.z, v.w * inv * gg.w);
      yr[c] = o;
    }
  }
}

void launch_rmsnorm(hipStream_t s, int cap_rows, const float* X, const float* g, uint16_t* Y,
                    const int32_t* n_rows, int d, float eps) {
  if (cap_rows <= 0) return;
  const dim3 grid((cap_rows + 3) / 4), blk(256);
  if (d == 1024) hipLaunchKernelGGL(k_rmsnorm<4>, grid, blk, 0, s, X, g, Y, n_rows, d, eps);
  else if (d == 2048) hipLaunchKernelGGL(k_rmsnorm<8>, grid, blk, 0, s, X, g, Y, n_rows, d, eps);
  else hipLaunchKernelGGL(k_rmsnorm<0>, grid, blk, 0, s, X, g, Y, n_rows, d, eps);
}

// ---------------------------------------------------------------------------
// Per-head RMSNorm of q and k (gain over head_dim) followed by the rotary
// embedding at each row's logical position, in place on the bf16 q|k|v row.
// Rotate-half layout: pair (i, i + hd/2) turns by pos * base^(-2i/hd); the
// cos/sin table is built on the host in double precision.  Each thread owns
// 8 consecutive dims (one 16-byte access); a head spans hd/8 threads and the
// rotation partner of thread t is thread t + hd/16 (fetched by shuffle).  A
// wave walks the heads of one row, so the row's table entries and the gains
// are read once per row rather than once per head.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_qk_rope(uint16_t* __restrict__ QKV, int ld,
                                                 const CallHeader* __restrict__ hdr,
                                                 const int32_t* __restrict__ pos,
                                                 const float* __restrict__ gq, const float* __restrict__ gk,
                                                 const float2* __restrict__ rope, int H, int Hkv, int hd,
                                                 float eps) {
  // one wave per row; lane = (head slot, thread t of the head); the cos/sin
  // of the row's position and the gains are loaded once and serve every head
  const int tph = hd >> 3;  // threads per head: 4, 8 or 16
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= hdr->T) return;
  const int lane = threadIdx.x & 63;
  const int t = lane % tph;
  const int slot = lane / tph;
  const int slots = 64 / tph;
  const int half_t = tph >> 1;
  const bool lo = t < half_t;
  const int i0 = (lo ? t : t - half_t) * 8;  // frequency index of dim 0 of this thread
  const float2* cs = rope + (size_t)pos[row] * (hd >> 1) + i0;
  float2 c[8];
  float g_q[8], g_k[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    c[e] = cs[e];
    g_q[e] = gq[t * 8 + e];
    g_k[e] = gk[t * 8 + e];
  }
  uint16_t* rowp = QKV + (size_t)row * ld;
  // The row is updated in place, so a head's load could not otherwise be
  // issued before the previous head's store: the heads' loads go out
  // together, kMaxIt at a time, then each head is normalised, rotated and
  // stored (heads are disjoint, and each element's arithmetic is unchanged).
  constexpr int kMaxIt = 8;
  auto head_ptr = [&](int head) {
    return rowp + (head < H ? head * hd : H * hd + (head - H) * hd) + t * 8;
  };
  for (int h0 = slot; h0 < H + Hkv; h0 += kMaxIt * slots) {
    uint4 vin[kMaxIt];
#pragma unroll
    for (int it = 0; it < kMaxIt; ++it) {
      const int head = h0 + it * slots;
      if (head < H + Hkv) vin[it] = *reinterpret_cast<const uint4*>(head_ptr(head));
    }
#pragma unroll
    for (int it = 0; it < kMaxIt; ++it) {
      const int head = h0 + it * slots;
      if (head >= H + Hkv) break;
      const bool isq = head < H;
      const uint4 v = vin[it];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16_to_f32((uint16_t)(w[e] & 0xffffu));
        x[2 * e + 1] = bf16_to_f32((uint16_t)(w[e] >> 16));
      }
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
      for (int m = tph >> 1; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, tph);
      const float inv = 1.0f / sqrtf(ss / (float)hd + eps);
      float y[8], q[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = x[e] * inv * (isq ? g_q[e] : g_k[e]);
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = __shfl_xor(y[e], half_t, tph);  // partner dims (i +- hd/2)
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // first half: x1 cos - x2 sin; second half: x2 cos + x1 sin
        o[e] = lo ? y[e] * c[e].x - q[e] * c[e].y : y[e] * c[e].x + q[e] * c[e].y;
      }
      uint4 out;
      out.x = pack_bf16x2(o[0], o[1]);
      out.y = pack_bf16x2(o[2], o[3]);
      out.z = pack_bf16x2(o[4], o[5]);
      out.w = pack_bf16x2(o[6], o[7]);
      *reinterpret_cast<uint4*>(head_ptr(head)) = out;
    }
  }
}

void launch_qk_rope(hipStream_t s, int cap_rows, uint16_t* QKV, int ld, const CallHeader* hdr,
                    const int32_t* pos, const float* gq, const float* gk, const float2* rope, int H,
                    int Hkv, int hd, float eps) {
  if (cap_rows <= 0) return;
  hipLaunchKernelGGL(k_qk_rope, dim3((unsigned)((cap_rows + 3) / 4)), dim3(256), 0, s, QKV, ld, hdr, pos, gq, gk,
                     rope, H, Hkv, hd, eps);
}

// ---------------------------------------------------------------------------
// Score head: s = w . RMSNorm_final(x) on the listed rows, fp32 throughout
// (shared linear head, "DuoLM: Fast and Effective Personalized Recommendation
// with Language Models", 核心方法).  Writes nothing when the gather flagged an
// out-of-range id.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_head(const float* __restrict__ X, DevBatch b,
                                              const float* __restrict__ gf, const float* __restrict__ w,
                                              float* __restrict__ scores, int d, float eps) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= b.hdr->n_scores || *b.err) return;
  const float* xr = X + (size_t)b.head_rows[i] * d;
  float ss = 0.f, dot = 0.f;
  for (int c = lane; c < (d >> 2); c += 64) {
    const float4 v = reinterpret_cast<const float4*>(xr)[c];
    const float4 gg = reinterpret_cast<const float4*>(gf)[c];
    const float4 ww = reinterpret_cast<const float4*>(w)[c];
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    dot += v.x * gg.x * ww.x + v.y * gg.y * ww.y + v.z * gg.z * ww.z + v.w * gg.w * ww.w;
  }
  ss = wave_sum(ss);
  dot = wave_sum(dot);
  if (lane == 0) scores[b.hdr->score_off + i] = dot / sqrtf(ss / (float)d + eps);
}

void launch_head(hipStream_t s, int cap_scores, const float* X, DevBatch b, const float* gf,
                 const float* w, float* scores, int d, float eps) {
  if (cap_scores <= 0) return;
  hipLaunchKernelGGL(k_head, dim3((cap_scores + 3) / 4), dim3(256), 0, s, X, b, gf, w, scores, d, eps);
}

// ---------------------------------------------------------------------------
// Session KV store: the K and V of each new prefix row of a session sequence
// go to row rho % kPageRows of its page rho / kPageRows, in the layer's block
// (an append to the cached prefix KV: "DuoLM: Fast and Effective Personalized
// Recommendation with Language Models", 未来方向 (3)).  One wave per row,
// 16 bytes per lane.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_kv_store(const uint16_t* __restrict__ QKV, int ld, DevBatch b, int H,
                                                  int Hkv, int hd) {
  const int T = b.hdr->T;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= T) return;
  const int n = b.hdr->n_seq;
  const int seg = packed_segment(b.seq_row_off, 2 * n, row);
  if (seg < n) return;  // a branch row
  const SeqDesc sd = b.seqs[seg - n];
  const int rho = row - sd.row_off;
  if (sd.pt < 0) return;  // not a session sequence
  const int kvw = Hkv * hd;
  const int pg = b.pages[sd.pt + rho / kPageRows];
  uint16_t* dst = b.kv + (int64_t)pg * b.page_stride + (size_t)(rho % kPageRows) * kvw;
  const uint16_t* src = QKV + (size_t)row * ld + H * hd;  // K then V, kvw values each
  for (int c = lane; c < kvw / 4; c += 64) {  // 16-byte chunks of K (first half) and V (second half)
    const bool isv = c >= kvw / 8;
    const int cc = isv ? c - kvw / 8 : c;
    const uint4 v = *reinterpret_cast<const uint4*>(src + (isv ? kvw : 0) + cc * 8);
    *reinterpret_cast<uint4*>(dst + (isv ? (size_t)kPageRows * kvw : 0) + cc * 8) = v;
  }
}

void launch_kv_store(hipStream_t s, int cap_rows, const uint16_t* QKV, int ld, DevBatch b, int H, int Hkv, int hd) {
  if (cap_rows <= 0) return;
  hipLaunchKernelGGL(k_kv_store, dim3((cap_rows + 3) / 4), dim3(256), 0, s, QKV, ld, b, H, Hkv, hd);
}

// ---------------------------------------------------------------------------
// Plain 16-byte copy (grid-stride), used to calibrate byte counters.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_copy(uint4* __restrict__ dst, const uint4* __restrict__ src, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) dst[i] = src[i];
}

void launch_copy(hipStream_t s, void* dst, const void* src, size_t nbytes) {
  const size_t n = nbytes / 16;
  if (n == 0) return;
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_copy, dim3((unsigned)blocks), dim3(256), 0, s, (uint4*)dst, (const uint4*)src, n);
}

// ---------------------------------------------------------------------------
// The call's scores to the caller's device buffer, unless the call-wide error
// flag is set (an out-of-range id leaves the caller's scores untouched).
// Enqueued behind the last launch, so the host waits once per call instead of
// reading the flag before it copies.  4-byte accesses: the caller's buffer
// need only be float-aligned.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_copy_scores(float* __restrict__ dst, const float* __restrict__ src, int n,
                                                     const int32_t* __restrict__ err) {
  if (*err) return;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) dst[i] = src[i];
}

void launch_copy_scores(hipStream_t s, float* dst, const float* src, int n, const int32_t* err) {
  if (n <= 0) return;
  const int blocks = std::min((n + 255) / 256, 1024);
  hipLaunchKernelGGL(k_copy_scores, dim3((unsigned)blocks), dim3(256), 0, s, dst, src, n, err);
}

// ---------------------------------------------------------------------------
// Fill n int32 values (clears flags with a kernel rather than a memset node).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_fill_i32(int32_t* __restrict__ p, int n, int32_t v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

void launch_fill_i32(hipStream_t s, int32_t* p, int n, int32_t v) {
  if (n <= 0) return;
  hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
}

}  // namespace duolm
