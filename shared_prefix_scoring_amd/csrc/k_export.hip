// Offline export of item vectors into the FP16 item table, and the reference
// scale it is calibrated against.
//
// The continuous-input interface turns an encoder representation a of an item
// into the ranker input z = e^gamma * rho * a / RMS(a): RMS normalisation,
// calibration by the reference scale rho of the ranker's native word
// embeddings, and a learnable gain e^gamma ("DuoLM: Fast and Effective
// Personalized Recommendation with Language Models", 一句话总结 and 核心方法;
// onedev.kr digest, 어떻게 동작하나).  After training every z is written once
// as FP16 into the GPU-resident table behind the virtual ids (same digest,
// 方法步骤详情 step 3).
//
// Both kernels stream HBM once.  Row statistics and the scaling run in fp64,
// so the only rounding that matters is the final one to binary16, done
// correctly (below).
#include "launch.h"

namespace duolm {

// IEEE binary16 round-to-nearest-even of a double in two hardware steps:
// round the double to float with round-to-odd (truncate toward zero, then set
// the last significand bit when anything was dropped), then convert that
// float to binary16 with the hardware's round-to-nearest-even.  Rounding to
// odd into a format with at least two more significand bits than the target
// (24 against 11 here, over binary16's whole exponent range) and then
// rounding to nearest gives exactly the single correct rounding (Boldo and
// Melquiond, "Emulation of FMA and correctly rounded sums: proved algorithms
// using rounding to odd", IEEE Trans. Computers 57(4), 2008).  The odd bit
// keeps a dropped remainder visible to the second rounding, so a value just
// off a binary16 tie is not mistaken for the tie.
__device__ __forceinline__ float f64_to_f32_odd(double x) {
  const float t = (float)x;  // nearest even
  const double back = (double)t;
  if (back == x) return t;   // exact
  uint32_t b = __float_as_uint(t);
  if (fabs(back) > fabs(x)) b -= 1u;  // rounded away from zero: step back to the truncation
  return __uint_as_float(b | 1u);
}

__device__ __forceinline__ uint32_t f64x2_to_f16x2_rne(double lo, double hi) {
  const _Float16 a = (_Float16)f64_to_f32_odd(lo), b = (_Float16)f64_to_f32_odd(hi);
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;  // every lane holds the same sum (each step adds the same pair)
}

// the values of one 16-byte chunk of the input row, widened exactly
template <int DT>
struct Chunk;
template <>
struct Chunk<EXPORT_F32> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void get(const uint4& v, double* o) {
    o[0] = (double)__uint_as_float(v.x);
    o[1] = (double)__uint_as_float(v.y);
    o[2] = (double)__uint_as_float(v.z);
    o[3] = (double)__uint_as_float(v.w);
  }
};
template <>
struct Chunk<EXPORT_BF16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void get(const uint4& v, double* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = (double)bf16_to_f32((uint16_t)(w[i] & 0xffffu));
      o[2 * i + 1] = (double)bf16_to_f32((uint16_t)(w[i] >> 16));
    }
  }
};
template <>
struct Chunk<EXPORT_F16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void get(const uint4& v, double* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = (double)f16_to_f32((uint16_t)(w[i] & 0xffffu));
      o[2 * i + 1] = (double)f16_to_f32((uint16_t)(w[i] >> 16));
    }
  }
};

// One 64-lane wave per row; lane l holds the row's 16-byte chunks l, l + 64,
// ... in registers (NQ of them), so the row is read from HBM exactly once.
template <int DT, int NQ>
__global__ __launch_bounds__(256) void k_export(const uint4* __restrict__ a, int64_t n_rows, int d,
                                                double scale, double eps, uint16_t* __restrict__ z) {
  using C = Chunk<DT>;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n_rows) return;
  const int nchunk = d / C::N;
  const uint4* src = a + row * nchunk;
  uint4 raw[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int c = lane + 64 * q;
    raw[q] = make_uint4(0, 0, 0, 0);
    if (c < nchunk) {  // streamed once: non-temporal
      const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + c));
      raw[q] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }
  // sum of squares in a fixed order: chunk by chunk within a lane, then the
  // wave butterfly (absent chunks hold zeros and add exactly nothing)
  double ss = 0.0;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    double v[C::N];
    C::get(raw[q], v);
#pragma unroll
    for (int i = 0; i < C::N; ++i) ss += v[i] * v[i];
  }
  ss = wave_sum_f64(ss);
  const double r = sqrt(ss / (double)d + eps);  // RMS(a)
  const double f = r > 0.0 ? scale / r : 0.0;   // an all-zero row with eps 0 exports as zeros
  uint16_t* dst = z + row * (int64_t)d;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int c = lane + 64 * q;
    if (c >= nchunk) continue;
    double v[C::N];
    C::get(raw[q], v);
    uint32_t h[C::N / 2];
#pragma unroll
    for (int i = 0; i < C::N / 2; ++i)
      h[i] = f64x2_to_f16x2_rne(v[2 * i] * f, v[2 * i + 1] * f);
    if constexpr (C::N == 8)
      reinterpret_cast<uint4*>(dst)[c] = make_uint4(h[0], h[1], h[2], h[3]);
    else
      reinterpret_cast<uint2*>(dst)[c] = make_uint2(h[0], h[1]);
  }
}

template <int DT>
static bool launch_export_dt(hipStream_t s, const void* a, int64_t n_rows, int d, double scale, double eps,
                             uint16_t* z) {
  const int per_lane = (d / Chunk<DT>::N + 63) / 64;
  const dim3 grid((unsigned)((n_rows + 3) / 4)), block(256);
  const uint4* src = (const uint4*)a;
#define EXPORT_CASE(nq)                                                                   \
  if (per_lane <= nq) {                                                                   \
    hipLaunchKernelGGL((k_export<DT, nq>), grid, block, 0, s, src, n_rows, d, scale, eps, z); \
    return true;                                                                          \
  }
  EXPORT_CASE(1)
  EXPORT_CASE(2)
  EXPORT_CASE(4)
  EXPORT_CASE(8)
  EXPORT_CASE(16)
  // 32 chunks per lane only where the widest row needs them (fp32 input):
  // 2-byte inputs reach kMaxExportDim at 16
  if constexpr (Chunk<DT>::N * 64 * 16 < kMaxExportDim) {
    EXPORT_CASE(32)
  }
#undef EXPORT_CASE
  return false;
}

bool launch_export(hipStream_t s, int dtype, const void* a, int64_t n_rows, int d, double scale, double eps,
                   uint16_t* z) {
  if (n_rows <= 0) return true;
  if (d < 8 || d % 8 || d > kMaxExportDim) return false;
  switch (dtype) {
    case EXPORT_F32: return launch_export_dt<EXPORT_F32>(s, a, n_rows, d, scale, eps, z);
    case EXPORT_BF16: return launch_export_dt<EXPORT_BF16>(s, a, n_rows, d, scale, eps, z);
    case EXPORT_F16: return launch_export_dt<EXPORT_F16>(s, a, n_rows, d, scale, eps, z);
    default: return false;
  }
}

// ---------------------------------------------------------------------------
// Reference scale rho = sqrt(mean of e^2 over every entry of the bf16 token
// embedding).  Block b sums its contiguous slice of 8-value chunks in fp64 in
// a fixed order and writes partial[b]; one block then adds the partials in
// index order.  The result does not depend on timing or on the launch.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double block_sum_f64(double v, double* sh) {
  v = wave_sum_f64(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  const double t = (sh[0] + sh[1]) + (sh[2] + sh[3]);
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(256) void k_sumsq_bf16(const uint4* __restrict__ E, int64_t n_chunks,
                                                    double* __restrict__ partial) {
  __shared__ double sh[4];
  const int64_t per = (n_chunks + gridDim.x - 1) / gridDim.x;
  const int64_t begin = (int64_t)blockIdx.x * per;
  const int64_t end = begin + per < n_chunks ? begin + per : n_chunks;
  double ss = 0.0;
  for (int64_t c = begin + threadIdx.x; c < end; c += 256) {
    double v[8];
    Chunk<EXPORT_BF16>::get(E[c], v);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
  }
  ss = block_sum_f64(ss, sh);
  if (threadIdx.x == 0) partial[blockIdx.x] = ss;
}

__global__ __launch_bounds__(256) void k_sumsq_final(const double* __restrict__ partial, int n_part,
                                                     double count, double* __restrict__ rho) {
  __shared__ double sh[4];
  double ss = 0.0;
  for (int i = threadIdx.x; i < n_part; i += 256) ss += partial[i];
  ss = block_sum_f64(ss, sh);
  if (threadIdx.x == 0) rho[0] = sqrt(ss / count);
}

void launch_reference_scale(hipStream_t s, const uint16_t* E, int64_t n_values, double* partial, double* rho) {
  hipLaunchKernelGGL(k_sumsq_bf16, dim3(kScaleBlocks), dim3(256), 0, s, (const uint4*)E, n_values / 8, partial);
  hipLaunchKernelGGL(k_sumsq_final, dim3(1), dim3(256), 0, s, (const double*)partial, kScaleBlocks,
                     (double)n_values, rho);
}

}  // namespace duolm
