// Host-side launchers of the HIP kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace duolm {

// Device views of one launch's batch description.
struct DevBatch {
  const CallHeader* hdr;
  const int32_t* seq_row_off;  // [2 n_seq + 1]: each sequence's first branch row, each one's first prefix row, T
  const SeqDesc* seqs;
  const WorkItem* pitems;
  const WorkItem* bitems;
  const int32_t* head_rows;
  int32_t* err;  // call-wide flag: nonzero after an out-of-range id
  // session KV pages (null when the call has no session sequences)
  const int32_t* pages;  // page tables of the call's session sequences
  uint16_t* kv;          // this layer's K/V block in page 0 of the pool
  int64_t page_stride;   // elements from one page to the next
};

// Grids are sized from host upper bounds ("cap" arguments); every kernel reads
// the true counts from the CallHeader and idles the surplus, so one captured
// graph serves any batch up to its caps.
void launch_embed(hipStream_t s, int cap_rows, const int32_t* ids, DevBatch b, const uint16_t* E,
                  const uint16_t* D, const uint16_t* Dinl, int V, int64_t n_vid, int d, float* X,
                  int32_t* pos);
// rows [0, *n_rows)
void launch_rmsnorm(hipStream_t s, int cap_rows, const float* X, const float* g, uint16_t* Y,
                    const int32_t* n_rows, int d, float eps);
void launch_qk_rope(hipStream_t s, int cap_rows, uint16_t* QKV, int ld, const CallHeader* hdr,
                    const int32_t* pos, const float* gq, const float* gk, const float2* rope, int H,
                    int Hkv, int hd, float eps);
void launch_head(hipStream_t s, int cap_scores, const float* X, DevBatch b, const float* gf,
                 const float* w, float* scores, int d, float eps);
void launch_copy(hipStream_t s, void* dst, const void* src, size_t nbytes);
// dst[0, n) = src[0, n) unless *err is nonzero
void launch_copy_scores(hipStream_t s, float* dst, const float* src, int n, const int32_t* err);
void launch_fill_i32(hipStream_t s, int32_t* p, int n, int32_t v);
// Store the K and V of the new prefix rows of session sequences into their
// pages (the layer's block, b.kv).  Rows of other sequences are skipped.
void launch_kv_store(hipStream_t s, int cap_rows, const uint16_t* QKV, int ld, DevBatch b, int H, int Hkv, int hd);

// GEMM epilogues
enum { EPI_BF16 = 0, EPI_RESID = 1, EPI_SWIGLU = 2 };
// C = epi(A[M,K] W[N,K]^T); M read from *dM (<= cap_m).  Returns false if the
// shape is unsupported (N % 64 or K % 64 nonzero).  share: launches running
// side by side on the chip (each counts 1/share of the CUs when the tile
// size is chosen).
bool launch_gemm(hipStream_t s, int epi, int cap_m, const uint16_t* A, int lda, const uint16_t* W,
                 int ldw, void* C, int ldc, const int32_t* dM, int N, int K, int share = 1);

// Attention over one launch's work items.  Returns rows covered per item.
int attn_rows_per_item(bool branch, int group);
bool attn_supported(int head_dim);
// cap_p prefix-tile blocks and cap_b branch-tile blocks in one launch (either may be 0).
void launch_attn(hipStream_t s, int hd, int cap_p, int cap_b, const uint16_t* QKV, int ld, uint16_t* O, int ldo,
                 DevBatch b, int H, int Hkv, float scale_log2);

// Offline export of encoder outputs a[n_rows, d] (16-byte aligned rows of
// dtype EXPORT_*) into FP16 rows z = scale * a / sqrt(mean(a^2) + eps).
// Returns false if d or dtype is unsupported.
enum { EXPORT_F32 = 0, EXPORT_BF16 = 1, EXPORT_F16 = 2 };
constexpr int kMaxExportDim = 8192;
bool launch_export(hipStream_t s, int dtype, const void* a, int64_t n_rows, int d, double scale, double eps,
                   uint16_t* z);
// rho = root mean square of n_values bf16 values (n_values % 8 == 0) into
// rho[0]; partial holds kScaleBlocks doubles of scratch.
constexpr int kScaleBlocks = 4096;
void launch_reference_scale(hipStream_t s, const uint16_t* E, int64_t n_values, double* partial, double* rho);

}  // namespace duolm
