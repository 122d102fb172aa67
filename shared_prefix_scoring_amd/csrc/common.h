// Shared definitions of the DuoLM MIS ranker library: the per-call batch
// descriptors that the host planner writes and the kernels read, and small
// device helpers.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace duolm {

// ---------------------------------------------------------------------------
// Batch description, uploaded once per forward launch.
//
// Rows of the activation buffers are packed in two regions: first the
// candidate-branch rows of every sequence, then the prefix rows of every
// sequence (so the last layer, whose prefix-row outputs nothing reads, can
// run its projections over the branch region [0, n_brows) alone).  A
// sequence has L causal rows (positions 0..L-1) and K candidate branches of M
// rows each (row i of a branch at position L + i, causal inside its branch);
// its prefix row rho sits at row_off + rho, its branch row rho (>= L) at
// boff + rho.
// MIS: one sequence per request.  Independent scoring: one sequence per
// (request, candidate) holding the prefix and that candidate alone (K = 1).
// Row rho of a sequence takes its id from ids[id_off + rho] when rho < id_len,
// else from ids[cand_id_off + rho - id_len].
//
// A session sequence continues a prefix whose first Lc rows were computed by
// earlier calls: their K and V live in pages of the KV pool (page table at
// pt), and only rows Lc .. of the sequence are packed.  row_off and id_off
// are then virtual (the packed position of row Lc, minus Lc), so row rho is
// still at row_off + rho; rows below Lc are never addressed in the packed
// buffers.  The prefix keys of such a sequence are read from its pages, into
// which the forward stores the K and V of its new prefix rows first.
// ---------------------------------------------------------------------------
struct SeqDesc {
  int32_t row_off;
  int32_t L;
  int32_t K;       // candidate branches
  int32_t id_off;
  int32_t id_len;
  int32_t cand_id_off;
  int32_t M;       // rows per candidate branch (positions L .. L + M - 1)
  int32_t pt;      // session sequences: offset of the page table in DevBatch::pages; else -1
  int32_t boff;    // branch row rho (>= L) is packed row boff + rho
  int32_t pad[3];
};

// A tile of query rows: prefix tiles start at row r0 of the sequence,
// branch tiles at candidate r0.  Carries its sequence's geometry so a
// workgroup needs one dependent load to start.
struct WorkItem {
  int32_t seq;
  int32_t r0;       // first row: prefix row r0, or branch row r0 (counted from row L; a branch start)
  int32_t row_off;  // query rows: item row rho of the sequence is packed row row_off + rho
  int32_t L;
  int32_t K;        // branch rows of the sequence (candidates x M)
  int32_t M;        // rows per candidate branch
  int32_t pt;       // the sequence's page table offset (-1: prefix keys are rows of the packed QKV)
  int32_t koff;     // prefix key rho is packed row koff + rho
};

struct CallHeader {
  int32_t T;         // rows in this launch
  int32_t n_seq;
  int32_t n_pitems;  // prefix attention tiles
  int32_t n_bitems;  // branch attention tiles
  int32_t n_scores;  // rows read by the score head
  int32_t score_off; // index of this launch's first score in the call's output
  int32_t n_inline;  // rows of the call's inline item-vector table (ids V+N .. V+N+n_inline-1)
  int32_t n_brows;   // rows of the branch region [0, n_brows)
  int32_t pad[8];
};
static_assert(sizeof(CallHeader) == 64, "header layout");

constexpr int kMaxPos = 32768;  // rotary table length; prefixes are shorter

// Session KV pages: kPageRows consecutive prefix rows of one sequence, for
// every layer: layer l holds K rows [kPageRows][Hkv * hd] then V rows, bf16.
// A page is one key tile of the attention kernel.
constexpr int kPageRows = 64;

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// The packed segment holding `row`: the last s < n_segs with start[s] <= row
// (start[] is non-decreasing; empty segments are skipped over).
__device__ __forceinline__ int packed_segment(const int32_t* __restrict__ start, int n_segs, int row) {
  int lo = 0, hi = n_segs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (start[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even: one v_cvt_pk_bf16_f32 per pair on gfx950
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, h);
  return (float)v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

}  // namespace duolm
