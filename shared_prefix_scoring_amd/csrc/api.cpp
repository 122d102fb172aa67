// C ABI and host executor of the DuoLM MIS ranker library.
//
// Per scoring call the executor
//   1. validates the request lengths (and, for host ids, the id ranges),
//   2. plans one or more forward launches: a launch is a set of sequences
//      packed row after row, with its causal-attention tiles, its branch
//      attention tiles and the rows the score head reads,
//   3. uploads each launch's small descriptor block (CallHeader, sequence
//      table, tile lists, head rows) from pinned memory,
//   4. runs the forward -- embedding gather, n_layers x (RMSNorm, QKV GEMM,
//      q/k norm + rotary, prefix attention, branch attention, O GEMM +
//      residual, RMSNorm, gate/up GEMM + SwiGLU, down GEMM + residual), score
//      head -- eagerly or by replaying a HIP graph captured for the launch's
//      shape bucket (every kernel reads its true sizes from the descriptor,
//      so only the descriptor and ids change between replays),
//   5. synchronises, checks the device id-range flag, and copies the scores.
#include <hip/hip_runtime.h>
#include <fcntl.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <set>
#include <string>
#include <thread>
#include <tuple>
#include <vector>

#include "../../include/duolm.h"
#include "../../include/duolm_debug.h"
#include "launch.h"

using namespace duolm;

// ---------------------------------------------------------------------------
// Scratch of duolm_score_batch_dev_noalloc: one fixed array per GPU, holding
// that entry point's activations, descriptor block and scores (each GPU the
// library runs on keeps it until the process ends).  In host code the name
// `scratch` is a host-side stand-in, not a device address: kernels and copies
// use the per-device address looked up once, with that device current, when a
// ranker is loaded on it (scratch_ptr below).
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(112) << 20;
constexpr size_t kScratchMetaBytes = size_t(1) << 20;  // the descriptor part (and its pinned staging)
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};


thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  // A failed runtime call (an allocation above all) leaves HIP's per-thread
  // last error set.  It is reported here; clear it, or the launch check of
  // the next call would report it again.
  if (code == DUOLM_ENOMEM || code == DUOLM_EHIP) (void)hipGetLastError();
  return code;
}

#define HIP_TRY(expr)                                                                \
  do {                                                                               \
    hipError_t e__ = (expr);                                                         \
    if (e__ != hipSuccess) return fail(DUOLM_EHIP, "%s: %s", #expr, hipGetErrorString(e__)); \
  } while (0)

constexpr int64_t kDefaultMaxRows = 262144;

// Calls of at least this many rows (and two sequences) run as two halves
// side by side, one per execution lane.
constexpr int64_t kLaneMinRows = 2048;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Bucket an upper bound: smallest m * 2^e >= x with m in [16, 32], so a
// graph's grids exceed the true sizes by at most 1/16 (the GEMM tile choice
// is made on these bounds).
int bucket(int x) {
  // small counts round to a power of two: a graph's grids are sized by these
  // caps, and each surplus attention workgroup still takes a CU slot to exit
  if (x <= 32) {
    int p = x <= 0 ? 0 : 1;
    while (p < x) p <<= 1;
    return p;
  }
  int e = 0;
  while ((x >> e) >= 32) ++e;
  int m = (x + (1 << e) - 1) >> e;
  return m << e;
}

struct LayerW {
  float* attn_norm;
  uint16_t* wqkv;
  float* q_norm;
  float* k_norm;
  uint16_t* wo;
  float* mlp_norm;
  uint16_t* wgu;
  uint16_t* wdown;
};

// One forward launch.
struct Plan {
  int T = 0;
  int TB = 0, TP = 0;  // rows of the branch region (packed first) and of the prefix region
  std::vector<int32_t> bstart, pstart;  // per sequence: first branch row, first prefix row (region-relative)
  std::vector<int32_t> seq_row_off;
  std::vector<SeqDesc> seqs;
  std::vector<WorkItem> pitems, bitems;
  std::vector<int32_t> head_rows;
  std::vector<int32_t> pages;   // page tables of session sequences
  std::vector<int32_t> cached;  // per sequence: prefix rows computed by earlier calls
  int score_off = 0;
  bool session = false;
};

struct Caps {
  int T, seq, pitems, bitems, scores, pages, session, brows;
  int share;  // launches of the call running side by side (GEMM tile choice)
  bool operator<(const Caps& o) const {
    return std::tie(T, seq, pitems, bitems, scores, pages, session, brows, share) <
           std::tie(o.T, o.seq, o.pitems, o.bitems, o.scores, o.pages, o.session, o.brows, o.share);
  }
};

struct Timed {
  int cls;
  hipEvent_t a, b;
  bool brows;  // the launch ran over the branch rows only (the last layer)
};

// A captured forward: one executable graph.  With profiling, every timed
// kernel is bracketed by event-record nodes added to the graph while it is
// captured (an event recorded on a capturing stream is not captured, but an
// explicit event-record node is, and times the nodes between its pair).  The
// events belong to the graph; each replay overwrites them.
struct GraphEntry {
  hipGraphExec_t exec = nullptr;
  std::vector<Timed> timed;
};

// One execution lane: an activation workspace, a descriptor block and a graph
// cache.  A large batch is split into two halves that run side by side on two
// streams -- each half's small and latency-bound kernels and the last partial
// round of its GEMMs leave CUs idle that the other half's kernels fill (a
// 64-request batch as two concurrent halves took 26.1 ms against 28.3 ms as
// one launch, measured with two handles).
constexpr int kLanes = 2;
struct Lane {
  hipStream_t stream = nullptr;  // lane 1: its own stream; lane 0 runs on the call's stream
  hipEvent_t done = nullptr;     // lane 1 finished the call's launches
  int cap_T = 0;
  void* ws = nullptr;
  float* X = nullptr;
  uint16_t* Xn = nullptr;
  uint16_t* QKV = nullptr;
  uint16_t* Ob = nullptr;
  uint16_t* Hb = nullptr;
  int32_t* pos = nullptr;
  int cap_seq = 0, cap_pi = 0, cap_bi = 0, cap_hs = 0, cap_pt = 0;
  size_t off_sro = 0, off_seq = 0, off_pi = 0, off_bi = 0, off_hr = 0, off_pt = 0, meta_bytes = 0;
  char* d_meta = nullptr;
  char* h_meta[2] = {nullptr, nullptr};
  hipEvent_t meta_free[2] = {nullptr, nullptr};
  int meta_slot = 0;
  std::map<Caps, GraphEntry> graphs;
};

}  // namespace

struct duolm_ranker {
  int device = 0;
  hipStream_t stream = nullptr;
  duolm_dims dims{};
  int nqkv = 0;  // (H + 2 Hkv) hd
  int64_t max_rows = kDefaultMaxRows;
  // weights
  void* wblob = nullptr;
  uint16_t* embed = nullptr;
  std::vector<LayerW> layers;
  float* final_norm = nullptr;
  float* head = nullptr;
  float2* rope = nullptr;
  uint16_t* vid = nullptr;
  int64_t n_vid = 0;
  // execution lanes: lane 0 runs on the call's stream, lane 1 on its own
  Lane lanes[kLanes];
  // the no-allocation entry point's lane: its buffers are carved from the
  // device's scratch per call; its pinned descriptor staging is made at load
  Lane na;
  hipEvent_t ids_ready = nullptr;  // the call's ids are on the device (lane 1 waits for it)
  hipEvent_t call_t0 = nullptr;    // timing origin of the call's timed launches
  // call inputs/outputs
  int64_t cap_ids = 0;
  int32_t* d_ids = nullptr;
  int64_t cap_out = 0;
  float* d_out = nullptr;
  int64_t cap_inline = 0;
  uint16_t* d_inline = nullptr;  // this call's inline item vectors (fp16 rows)
  int32_t call_n_inline = 0;
  int32_t* d_err = nullptr;
  int32_t* h_err = nullptr;  // pinned
  char* h_stage = nullptr;   // pinned staging for host ids in and host scores out
  size_t cap_stage = 0;
  // session KV pool: kv_pages pages of kPageRows prefix rows, all layers
  uint16_t* kv_pool = nullptr;
  int64_t kv_pages = 0;
  int64_t page_elems = 0;
  std::vector<int32_t> kv_free;  // free page indices (a stack)
  std::set<duolm_session*> sessions;
  // profiling
  uint32_t prof_mask = 0;
  duolm_kernel_stats stats[DUOLM_K_COUNT]{};
  std::vector<hipEvent_t> ev_pool;
  size_t ev_used = 0;
};

// A user session: a prefix whose K and V stay in the ranker's KV pool between
// calls, so new history rows are appended without recomputing the old ones.
struct duolm_session {
  duolm_ranker* owner;
  int32_t L = 0;               // prefix rows computed so far
  std::vector<int32_t> pages;  // page i holds rows [i kPageRows, (i + 1) kPageRows)
};

namespace {

// ---------------------------------------------------------------------------
// weights file
// ---------------------------------------------------------------------------
struct FileHeader {
  char magic[8];
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ffn, vocab;
  float rms_eps, rope_base;
  uint32_t reserved[5];
};
static_assert(sizeof(FileHeader) == 64, "file header");

int check_dims(const FileHeader& h) {
  if (memcmp(h.magic, "DUOLMW01", 8) != 0) return fail(DUOLM_EIO, "bad magic");
  if (h.n_layers < 1 || h.d_model < 64 || h.n_heads < 1 || h.n_kv_heads < 1 || h.d_ffn < 32 || h.vocab < 1)
    return fail(DUOLM_EINVAL, "bad dimensions in header");
  if (h.n_heads % h.n_kv_heads != 0) return fail(DUOLM_EINVAL, "n_heads %% n_kv_heads != 0");
  const int G = h.n_heads / h.n_kv_heads;
  // the attention kernel keeps the rows' own K and V in the query block's
  // LDS, which holds them only with at least two query heads per KV head
  if (G < 2 || G > 16 || 16 % G != 0)
    return fail(DUOLM_EINVAL, "query heads per KV head must be 2, 4, 8 or 16");
  if (!attn_supported(h.head_dim)) return fail(DUOLM_EINVAL, "head_dim must be 32, 64 or 128");
  if (h.d_model % 64 || h.d_ffn % 64 || (h.n_heads * h.head_dim) % 64)
    return fail(DUOLM_EINVAL, "d_model, d_ffn and n_heads*head_dim must be multiples of 64");
  if (!(h.rms_eps >= 0.f) || !(h.rope_base > 1.f)) return fail(DUOLM_EINVAL, "bad eps / rope base");
  return DUOLM_OK;
}

struct SrcTensor {
  const void* p;
  size_t bytes;
};

int parse_tensors(const FileHeader& h, const char* base, uint64_t nbytes, std::vector<SrcTensor>& out) {
  const size_t d = h.d_model, hq = h.n_heads, hk = h.n_kv_heads, hd = h.head_dim, f = h.d_ffn;
  std::vector<size_t> sizes;
  sizes.push_back((size_t)h.vocab * d * 2);
  for (int l = 0; l < h.n_layers; ++l) {
    sizes.push_back(d * 4);            // attn_norm
    sizes.push_back(hq * hd * d * 2);  // wq
    sizes.push_back(hk * hd * d * 2);  // wk
    sizes.push_back(hk * hd * d * 2);  // wv
    sizes.push_back(hd * 4);           // q_norm
    sizes.push_back(hd * 4);           // k_norm
    sizes.push_back(d * hq * hd * 2);  // wo
    sizes.push_back(d * 4);            // mlp_norm
    sizes.push_back(f * d * 2);        // w_gate
    sizes.push_back(f * d * 2);        // w_up
    sizes.push_back(d * f * 2);        // w_down
  }
  sizes.push_back(d * 4);  // final_norm
  sizes.push_back(d * 4);  // head
  size_t off = 64;
  out.clear();
  for (size_t s : sizes) {
    off = align_up(off, 64);
    if (off + s > nbytes) return fail(DUOLM_EIO, "weights blob too short (%llu bytes)", (unsigned long long)nbytes);
    out.push_back({base + off, s});
    off += s;
  }
  return DUOLM_OK;
}

// Build the device weight image.  Q/K/V rows are concatenated into one
// [(H + 2 Hkv) hd, d] matrix; gate and up rows are interleaved in 32-row
// blocks (gate block p, up block p) so the gate/up GEMM's epilogue finds each
// output column's gate and up values in the same lane.
int load_weights(duolm_ranker* R, const FileHeader& h, const std::vector<SrcTensor>& src) {
  const size_t d = h.d_model, hq = h.n_heads, hk = h.n_kv_heads, hd = h.head_dim, f = h.d_ffn;
  const size_t nqkv = (hq + 2 * hk) * hd;
  auto a = [](size_t x) { return align_up(x, 256); };
  size_t total = a((size_t)h.vocab * d * 2);
  const size_t per_layer = a(d * 4) + a(nqkv * d * 2) + a(hd * 4) * 2 + a(d * hq * hd * 2) + a(d * 4) +
                           a(2 * f * d * 2) + a(d * f * 2);
  total += per_layer * h.n_layers + a(d * 4) * 2 + a((size_t)kMaxPos * (hd / 2) * sizeof(float2));
  HIP_TRY(hipMalloc(&R->wblob, total));
  char* p = (char*)R->wblob;
  auto take = [&](size_t bytes) {
    char* q = p;
    p += a(bytes);
    return q;
  };
  size_t ti = 0;
  R->embed = (uint16_t*)take((size_t)h.vocab * d * 2);
  HIP_TRY(hipMemcpy(R->embed, src[ti].p, src[ti].bytes, hipMemcpyHostToDevice));
  ++ti;
  R->layers.resize(h.n_layers);
  for (int l = 0; l < h.n_layers; ++l) {
    LayerW& W = R->layers[l];
    W.attn_norm = (float*)take(d * 4);
    W.wqkv = (uint16_t*)take(nqkv * d * 2);
    W.q_norm = (float*)take(hd * 4);
    W.k_norm = (float*)take(hd * 4);
    W.wo = (uint16_t*)take(d * hq * hd * 2);
    W.mlp_norm = (float*)take(d * 4);
    W.wgu = (uint16_t*)take(2 * f * d * 2);
    W.wdown = (uint16_t*)take(d * f * 2);
    HIP_TRY(hipMemcpy(W.attn_norm, src[ti].p, src[ti].bytes, hipMemcpyHostToDevice));
    ++ti;
    char* q = (char*)W.wqkv;
    for (int k = 0; k < 3; ++k) {  // wq, wk, wv
      HIP_TRY(hipMemcpy(q, src[ti].p, src[ti].bytes, hipMemcpyHostToDevice));
      q += src[ti].bytes;
      ++ti;
    }
    HIP_TRY(hipMemcpy(W.q_norm, src[ti].p, src[ti].bytes, hipMemcpyHostToDevice));
    ++ti;
    HIP_TRY(hipMemcpy(W.k_norm, src[ti].p, src[ti].bytes, hipMemcpyHostToDevice));
    ++ti;
    HIP_TRY(hipMemcpy(W.wo, src[ti].p, src[ti].bytes, hipMemcpyHostToDevice));
    ++ti;
    HIP_TRY(hipMemcpy(W.mlp_norm, src[ti].p, src[ti].bytes, hipMemcpyHostToDevice));
    ++ti;
    const size_t blk = 32 * d * 2;  // bytes of a 32-row block
    // gate block p -> rows [64p, 64p + 32), up block p -> rows [64p + 32, 64p + 64)
    HIP_TRY(hipMemcpy2D(W.wgu, 2 * blk, src[ti].p, blk, blk, f / 32, hipMemcpyHostToDevice));
    ++ti;
    HIP_TRY(hipMemcpy2D((char*)W.wgu + blk, 2 * blk, src[ti].p, blk, blk, f / 32, hipMemcpyHostToDevice));
    ++ti;
    HIP_TRY(hipMemcpy(W.wdown, src[ti].p, src[ti].bytes, hipMemcpyHostToDevice));
    ++ti;
  }
  R->final_norm = (float*)take(d * 4);
  HIP_TRY(hipMemcpy(R->final_norm, src[ti].p, src[ti].bytes, hipMemcpyHostToDevice));
  ++ti;
  R->head = (float*)take(d * 4);
  HIP_TRY(hipMemcpy(R->head, src[ti].p, src[ti].bytes, hipMemcpyHostToDevice));
  ++ti;
  // rotary table: angle = pos * base^(-2i/hd), computed in double
  const size_t half = hd / 2;
  std::vector<float2> tab((size_t)kMaxPos * half);
  for (size_t i = 0; i < half; ++i) {
    const double inv_freq = std::pow((double)h.rope_base, -2.0 * (double)i / (double)hd);
    for (int pp = 0; pp < kMaxPos; ++pp) {
      const double ang = (double)pp * inv_freq;
      tab[(size_t)pp * half + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
    }
  }
  R->rope = (float2*)take(tab.size() * sizeof(float2));
  HIP_TRY(hipMemcpy(R->rope, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice));
  return DUOLM_OK;
}

int create_from_blob(const void* blob, uint64_t nbytes, int dev, duolm_ranker** out) {
  if (!blob || !out) return fail(DUOLM_EINVAL, "NULL argument");
  if (nbytes < sizeof(FileHeader)) return fail(DUOLM_EIO, "weights blob shorter than its header");
  FileHeader h;
  memcpy(&h, blob, sizeof(h));
  int rc = check_dims(h);
  if (rc) return rc;
  std::vector<SrcTensor> src;
  rc = parse_tensors(h, (const char*)blob, nbytes, src);
  if (rc) return rc;
  int ndev = 0;
  HIP_TRY(hipGetDeviceCount(&ndev));
  if (dev < 0 || dev >= ndev) return fail(DUOLM_EINVAL, "hip_device %d out of range (%d devices)", dev, ndev);
  HIP_TRY(hipSetDevice(dev));
  duolm_ranker* R = new duolm_ranker();
  R->device = dev;
  R->dims.n_layers = h.n_layers;
  R->dims.d_model = h.d_model;
  R->dims.n_heads = h.n_heads;
  R->dims.n_kv_heads = h.n_kv_heads;
  R->dims.head_dim = h.head_dim;
  R->dims.d_ffn = h.d_ffn;
  R->dims.vocab = h.vocab;
  R->dims.rms_eps = h.rms_eps;
  R->dims.rope_base = h.rope_base;
  R->dims.max_prefix = kMaxPos - 1;
  R->nqkv = (h.n_heads + 2 * h.n_kv_heads) * h.head_dim;
  if (const char* e = getenv("DUOLM_MAX_ROWS")) {
    const long v = atol(e);
    if (v >= 1024) R->max_rows = v;
  }
  R->dims.max_rows = (int32_t)R->max_rows;
  rc = load_weights(R, h, src);
  if (rc == DUOLM_OK) {
    hipError_t e = hipStreamCreateWithFlags(&R->stream, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipHostMalloc((void**)&R->h_err, sizeof(int32_t));
    if (e == hipSuccess) e = hipMalloc((void**)&R->d_err, sizeof(int32_t));
    if (e == hipSuccess) e = hipEventCreateWithFlags(&R->ids_ready, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreate(&R->call_t0);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&R->na.meta_free[0], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&R->na.meta_free[1], hipEventDisableTiming);
    if (e == hipSuccess) e = hipHostMalloc((void**)&R->na.h_meta[0], kScratchMetaBytes);
    if (e == hipSuccess) e = hipHostMalloc((void**)&R->na.h_meta[1], kScratchMetaBytes);
    for (int li = 0; li < kLanes && e == hipSuccess; ++li) {
      Lane& Ln = R->lanes[li];
      e = hipEventCreateWithFlags(&Ln.meta_free[0], hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&Ln.meta_free[1], hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&Ln.done, hipEventDisableTiming);
      if (e == hipSuccess && li > 0) e = hipStreamCreateWithFlags(&Ln.stream, hipStreamNonBlocking);
    }
    if (e != hipSuccess) rc = fail(DUOLM_EHIP, "stream/event setup: %s", hipGetErrorString(e));
  }
  if (rc == DUOLM_OK && dev < kMaxDevices) {
    // the scratch's address on this device, once per device (this device is current)
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) rc = fail(DUOLM_EHIP, "scratch address on device %d: %s", dev, hipGetErrorString(e));
      else g_scratch_ptr[dev] = p;
    }
  }
  if (rc != DUOLM_OK) {
    duolm_free_ranker(R);
    return rc;
  }
  *out = R;
  return DUOLM_OK;
}

// ---------------------------------------------------------------------------
// capacities
// ---------------------------------------------------------------------------
void free_graph(GraphEntry& ge) {
  if (ge.exec) (void)hipGraphExecDestroy(ge.exec);
  ge.exec = nullptr;
  for (const Timed& t : ge.timed) {
    (void)hipEventDestroy(t.a);
    (void)hipEventDestroy(t.b);
  }
  ge.timed.clear();
}

void drop_graphs(duolm_ranker* R) {
  for (Lane& Ln : R->lanes) {
    for (auto& kv : Ln.graphs) free_graph(kv.second);
    Ln.graphs.clear();
  }
}

// wait for everything in flight on the handle's streams
int sync_all(duolm_ranker* R) {
  HIP_TRY(hipStreamSynchronize(R->stream));
  for (Lane& Ln : R->lanes)
    if (Ln.stream) HIP_TRY(hipStreamSynchronize(Ln.stream));
  return DUOLM_OK;
}

int ensure_rows(duolm_ranker* R, Lane& Ln, int T) {
  if (T <= Ln.cap_T) return DUOLM_OK;
  int rc = sync_all(R);
  if (rc) return rc;
  drop_graphs(R);
  if (Ln.ws) (void)hipFree(Ln.ws);
  Ln.ws = nullptr;
  Ln.cap_T = 0;
  const int cap = (int)std::min<int64_t>(R->max_rows, std::max<int64_t>(4096, align_up((size_t)T + T / 4, 4096)));
  const auto& D = R->dims;
  auto a = [](size_t x) { return align_up(x, 256); };
  const size_t bX = a((size_t)cap * D.d_model * 4), bXn = a((size_t)cap * D.d_model * 2),
               bQ = a((size_t)cap * R->nqkv * 2), bO = a((size_t)cap * D.n_heads * D.head_dim * 2),
               bH = a((size_t)cap * D.d_ffn * 2), bP = a((size_t)cap * 4);
  hipError_t e = hipMalloc(&Ln.ws, bX + bXn + bQ + bO + bH + bP);
  if (e != hipSuccess) return fail(DUOLM_ENOMEM, "workspace for %d rows: %s", cap, hipGetErrorString(e));
  char* p = (char*)Ln.ws;
  Ln.X = (float*)p; p += bX;
  Ln.Xn = (uint16_t*)p; p += bXn;
  Ln.QKV = (uint16_t*)p; p += bQ;
  Ln.Ob = (uint16_t*)p; p += bO;
  Ln.Hb = (uint16_t*)p; p += bH;
  Ln.pos = (int32_t*)p;
  Ln.cap_T = cap;
  return DUOLM_OK;
}

int ensure_meta(duolm_ranker* R, Lane& Ln, int n_seq, int n_pi, int n_bi, int n_hs, int n_pt) {
  if (n_seq <= Ln.cap_seq && n_pi <= Ln.cap_pi && n_bi <= Ln.cap_bi && n_hs <= Ln.cap_hs && n_pt <= Ln.cap_pt)
    return DUOLM_OK;
  int rc = sync_all(R);
  if (rc) return rc;
  drop_graphs(R);
  auto grow = [](int need, int have) { return std::max(have, std::max(256, (int)align_up((size_t)need * 5 / 4, 256))); };
  Ln.cap_seq = grow(n_seq, Ln.cap_seq);
  Ln.cap_pi = grow(n_pi, Ln.cap_pi);
  Ln.cap_bi = grow(n_bi, Ln.cap_bi);
  Ln.cap_hs = grow(n_hs, Ln.cap_hs);
  Ln.cap_pt = grow(n_pt, Ln.cap_pt);
  size_t off = align_up(sizeof(CallHeader), 256);
  Ln.off_sro = off; off = align_up(off + (size_t)(2 * Ln.cap_seq + 1) * 4, 256);
  Ln.off_seq = off; off = align_up(off + (size_t)Ln.cap_seq * sizeof(SeqDesc), 256);
  Ln.off_pi = off; off = align_up(off + (size_t)Ln.cap_pi * sizeof(WorkItem), 256);
  Ln.off_bi = off; off = align_up(off + (size_t)Ln.cap_bi * sizeof(WorkItem), 256);
  Ln.off_hr = off; off = align_up(off + (size_t)Ln.cap_hs * 4, 256);
  Ln.off_pt = off; off = align_up(off + (size_t)Ln.cap_pt * 4, 256);
  Ln.meta_bytes = off;
  if (Ln.d_meta) (void)hipFree(Ln.d_meta);
  for (auto& h : Ln.h_meta)
    if (h) (void)hipHostFree(h);
  Ln.d_meta = nullptr;
  Ln.h_meta[0] = Ln.h_meta[1] = nullptr;
  if (hipMalloc((void**)&Ln.d_meta, off) != hipSuccess || hipHostMalloc((void**)&Ln.h_meta[0], off) != hipSuccess ||
      hipHostMalloc((void**)&Ln.h_meta[1], off) != hipSuccess) {
    Ln.cap_seq = Ln.cap_pi = Ln.cap_bi = Ln.cap_hs = Ln.cap_pt = 0;
    return fail(DUOLM_ENOMEM, "descriptor buffers (%zu bytes)", off);
  }
  return DUOLM_OK;
}

// Grow a device buffer.  Captured graphs bake buffer addresses, so a
// reallocation drops them.
template <typename Tp>
int ensure_buf(duolm_ranker* R, Tp*& ptr, int64_t& cap, int64_t need) {
  if (need <= cap) return DUOLM_OK;
  int rc = sync_all(R);
  if (rc) return rc;
  drop_graphs(R);
  if (ptr) (void)hipFree(ptr);
  ptr = nullptr;
  cap = 0;
  const int64_t n = std::max<int64_t>(need + need / 4, 4096);
  if (hipMalloc((void**)&ptr, (size_t)n * sizeof(Tp)) != hipSuccess) return fail(DUOLM_ENOMEM, "device buffer");
  cap = n;
  return DUOLM_OK;
}

DevBatch dev_batch(duolm_ranker* R, const Lane& Ln) {
  DevBatch b;
  b.hdr = (const CallHeader*)Ln.d_meta;
  b.seq_row_off = (const int32_t*)(Ln.d_meta + Ln.off_sro);
  b.seqs = (const SeqDesc*)(Ln.d_meta + Ln.off_seq);
  b.pitems = (const WorkItem*)(Ln.d_meta + Ln.off_pi);
  b.bitems = (const WorkItem*)(Ln.d_meta + Ln.off_bi);
  b.head_rows = (const int32_t*)(Ln.d_meta + Ln.off_hr);
  b.err = R->d_err;
  b.pages = (const int32_t*)(Ln.d_meta + Ln.off_pt);
  b.kv = R->kv_pool;
  b.page_stride = R->page_elems;
  return b;
}

// ---------------------------------------------------------------------------
// planning
// ---------------------------------------------------------------------------
// A sequence: L causal rows, then K candidate branches of M rows each.
// Branch attention tiles hold whole branches (a branch row's in-branch keys
// are rows of its own tile); the score head reads each branch's last row.
// Branch rows go to the branch region, prefix rows to the prefix region that
// follows it; prefix-side offsets are region-relative until plan_close adds
// the branch region's size.
void plan_add_seq(duolm_ranker* R, Plan& P, int L, int K, int M, int id_off, int id_len, int cand_id_off) {
  const int G = R->dims.n_heads / R->dims.n_kv_heads;
  const int s = (int)P.seqs.size();
  const int KM = K * M;
  SeqDesc sd{};
  sd.row_off = P.TP;
  sd.boff = P.TB - L;
  sd.L = L;
  sd.K = K;
  sd.id_off = id_off;
  sd.id_len = id_len;
  sd.cand_id_off = cand_id_off;
  sd.M = M;
  sd.pt = -1;
  P.seqs.push_back(sd);
  P.cached.push_back(0);
  P.pstart.push_back(P.TP);
  P.bstart.push_back(P.TB);
  const int rp = attn_rows_per_item(false, G);
  const int rb = attn_rows_per_item(true, G) / M * M;  // whole branches per tile
  for (int r0 = 0; r0 < L; r0 += rp) P.pitems.push_back({s, r0, sd.row_off, L, KM, M, -1, sd.row_off});
  for (int c0 = 0; c0 < KM; c0 += rb) P.bitems.push_back({s, c0, sd.boff, L, KM, M, -1, sd.row_off});
  for (int j = 0; j < K; ++j) P.head_rows.push_back(P.TB + j * M + M - 1);
  P.TP += L;
  P.TB += KM;
  P.T += L + KM;
}

// A session sequence: prefix rows [0, Lc) were computed by earlier calls (their
// K and V are in the session's pages), rows [Lc, L) are new, then K branches.
// Only the new rows and the branches are packed; row_off and id_off are
// virtual (row Lc sits at the prefix region's next row).  ids: the new prefix
// ids at new_id_off, the candidates' at cand_id_off.
void plan_add_session(duolm_ranker* R, Plan& P, int Lc, int L, int K, int M, int new_id_off, int cand_id_off,
                      const std::vector<int32_t>& pages) {
  const int G = R->dims.n_heads / R->dims.n_kv_heads;
  const int s = (int)P.seqs.size();
  const int KM = K * M;
  SeqDesc sd{};
  sd.row_off = P.TP - Lc;
  sd.boff = P.TB - L;
  sd.L = L;
  sd.K = K;
  sd.id_off = new_id_off - Lc;
  sd.id_len = L;
  sd.cand_id_off = cand_id_off;
  sd.M = M;
  sd.pt = (int)P.pages.size();
  P.pages.insert(P.pages.end(), pages.begin(), pages.begin() + (L + kPageRows - 1) / kPageRows);
  P.seqs.push_back(sd);
  P.cached.push_back(Lc);
  P.pstart.push_back(P.TP);
  P.bstart.push_back(P.TB);
  const int rp = attn_rows_per_item(false, G);
  const int rb = attn_rows_per_item(true, G) / M * M;
  for (int r0 = Lc; r0 < L; r0 += rp) P.pitems.push_back({s, r0, sd.row_off, L, KM, M, sd.pt, sd.row_off});
  for (int c0 = 0; c0 < KM; c0 += rb) P.bitems.push_back({s, c0, sd.boff, L, KM, M, sd.pt, sd.row_off});
  for (int j = 0; j < K; ++j) P.head_rows.push_back(P.TB + j * M + M - 1);
  P.TP += L - Lc;
  P.TB += KM;
  P.T += (L - Lc) + KM;
  P.session = true;
}

// Close a launch: place the prefix region after the branch region, build the
// row-to-segment table, and order the attention tiles longest first (their
// key count is the work), so the grid's tail is made of short tiles.
void plan_close(duolm_ranker* R, Plan& P) {
  const int TB = P.TB;
  for (SeqDesc& sd : P.seqs) sd.row_off += TB;
  for (WorkItem& w : P.pitems) {
    w.row_off += TB;
    w.koff += TB;
  }
  for (WorkItem& w : P.bitems) w.koff += TB;
  P.seq_row_off.assign(P.bstart.begin(), P.bstart.end());
  for (int32_t p : P.pstart) P.seq_row_off.push_back(TB + p);
  P.seq_row_off.push_back(P.T);
  const int G = R->dims.n_heads / R->dims.n_kv_heads;
  const int rp = attn_rows_per_item(false, G);
  auto pkeys = [&](const WorkItem& w) { return std::min(w.r0 + rp, w.L); };
  std::stable_sort(P.pitems.begin(), P.pitems.end(),
                   [&](const WorkItem& a, const WorkItem& b) { return pkeys(a) > pkeys(b); });
  std::stable_sort(P.bitems.begin(), P.bitems.end(),
                   [&](const WorkItem& a, const WorkItem& b) { return a.L > b.L; });
}

// Algorithmic FLOPs and bytes of one launch per kernel class.
// rows: the rows a row-wise launch covers (all T, or the branch rows of the
// last layer).
void launch_work(const duolm_ranker* R, const Plan& P, double fl[DUOLM_K_COUNT], double by[DUOLM_K_COUNT],
                 double rows) {
  const auto& D = R->dims;
  const double T = rows, d = D.d_model, H = D.n_heads, Hk = D.n_kv_heads, hd = D.head_dim, F = D.d_ffn;
  const double nq = R->nqkv;
  for (int i = 0; i < DUOLM_K_COUNT; ++i) fl[i] = by[i] = 0;
  by[DUOLM_K_EMBED] = T * (d * 2 + d * 4 + 8);
  fl[DUOLM_K_RMSNORM] = T * d * 4;
  by[DUOLM_K_RMSNORM] = T * (d * 4 + d * 2);
  fl[DUOLM_K_GEMM_QKV] = 2 * T * d * nq;
  by[DUOLM_K_GEMM_QKV] = (nq * d + T * d + T * nq) * 2;
  by[DUOLM_K_QK_ROPE] = T * (H + Hk) * hd * 4 + T * 4;
  fl[DUOLM_K_GEMM_O] = 2 * T * H * hd * d;
  by[DUOLM_K_GEMM_O] = (d * H * hd + T * H * hd) * 2 + T * d * 8;
  fl[DUOLM_K_GEMM_GATEUP] = 2 * T * d * 2 * F;
  by[DUOLM_K_GEMM_GATEUP] = (2 * F * d + T * d + T * F) * 2;
  fl[DUOLM_K_GEMM_DOWN] = 2 * T * F * d;
  by[DUOLM_K_GEMM_DOWN] = (d * F + T * F) * 2 + T * d * 8;
  for (size_t i = 0; i < P.seqs.size(); ++i) {
    const SeqDesc& s = P.seqs[i];
    const double L = s.L, K = s.K, M = s.M, Lc = P.cached[i];
    // new causal rows r = Lc .. L - 1 see r + 1 keys; cached rows' K/V come from pages
    fl[DUOLM_K_ATTN_PREFIX] += 4 * hd * H * (L * (L + 1) - Lc * (Lc + 1)) / 2;
    if (L > Lc) by[DUOLM_K_ATTN_PREFIX] += (L - Lc) * (H * hd * 2 + Hk * hd * 4 + H * hd * 2) + Lc * Hk * hd * 4;
    // branch row i sees L prefix keys and i + 1 keys of its own branch
    fl[DUOLM_K_ATTN_BRANCH] += 4 * hd * H * K * (M * L + M * (M + 1) / 2);
    if (K > 0) by[DUOLM_K_ATTN_BRANCH] += L * Hk * hd * 4 + K * M * (H * hd * 2 + Hk * hd * 4 + H * hd * 2);
  }
  by[DUOLM_K_HEAD] = (double)P.head_rows.size() * (d * 4 + 4);
  fl[DUOLM_K_HEAD] = (double)P.head_rows.size() * d * 4;
}

// ---------------------------------------------------------------------------
// forward enqueue
// ---------------------------------------------------------------------------
hipEvent_t pool_event(duolm_ranker* R) {
  if (R->ev_used == R->ev_pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    R->ev_pool.push_back(e);
  }
  return R->ev_pool[R->ev_used++];
}

struct Enq {
  duolm_ranker* R;
  Lane* ln;
  hipStream_t s;
  std::vector<Timed>* timed;  // eager: where to record timing events (null: no timing)
  GraphEntry* capture;        // graph capture in progress (null: eager)
  const int32_t* ids = nullptr;  // the call's ids on the device (null: the handle's id buffer)
  float* out = nullptr;          // where the head writes the scores (null: the handle's score buffer)
  int stop_layer = -1, stop_stage = -1;
  bool stopped = false;
  bool brows = false;  // the launches being enqueued cover the branch rows only
  hipError_t cap_err = hipSuccess;

  void note(hipError_t e) {
    if (e != hipSuccess && cap_err == hipSuccess) cap_err = e;
  }
  // append an event-record node after everything captured so far
  void record_node(hipEvent_t ev) {
    hipStreamCaptureStatus st;
    unsigned long long id = 0;
    hipGraph_t g = nullptr;
    const hipGraphNode_t* deps = nullptr;
    size_t nd = 0;
    hipError_t e = hipStreamGetCaptureInfo_v2(s, &st, &id, &g, &deps, &nd);
    hipGraphNode_t n = nullptr;
    if (e == hipSuccess) e = hipGraphAddEventRecordNode(&n, g, deps, nd, ev);
    if (e == hipSuccess) e = hipStreamUpdateCaptureDependencies(s, &n, 1, hipStreamSetCaptureDependencies);
    note(e);
  }

  template <typename F>
  void run(int cls, F&& f) {
    const bool want = R->prof_mask >> cls & 1u;
    if (capture && want) {  // bracket the kernel with event-record nodes
      hipEvent_t a = nullptr, b = nullptr;
      note(hipEventCreate(&a));
      note(hipEventCreate(&b));
      if (cap_err != hipSuccess) {
        if (a) (void)hipEventDestroy(a);
        if (b) (void)hipEventDestroy(b);
        f();
        return;
      }
      capture->timed.push_back({cls, a, b, brows});
      record_node(a);
      f();
      record_node(b);
      return;
    }
    if (!capture && timed && want) {
      hipEvent_t a = pool_event(R), b = pool_event(R);
      if (a && b) {
        (void)hipEventRecord(a, s);
        f();
        (void)hipEventRecord(b, s);
        timed->push_back({cls, a, b, brows});
        return;
      }
    }
    f();
  }
  bool stop(int layer, int stage) {
    if (layer == stop_layer && stage == stop_stage) stopped = true;
    return stopped;
  }
};

void enqueue_forward(Enq& q, const Caps& c) {
  duolm_ranker* R = q.R;
  const auto& D = R->dims;
  const int d = D.d_model, H = D.n_heads, Hk = D.n_kv_heads, hd = D.head_dim, F = D.d_ffn, nq = R->nqkv;
  const float eps = D.rms_eps;
  const float scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)hd));
  hipStream_t s = q.s;
  Lane* ln = q.ln;
  DevBatch b = dev_batch(R, *ln);
  const int32_t* dT = &b.hdr->T;
  const int32_t* dB = &b.hdr->n_brows;
  const int32_t* ids = q.ids ? q.ids : R->d_ids;
  float* scores = q.out ? q.out : R->d_out;
  q.run(DUOLM_K_EMBED, [&] { launch_embed(s, c.T, ids, b, R->embed, R->vid, R->d_inline, D.vocab, R->n_vid, d, ln->X, ln->pos); });
  if (q.stop(0, DUOLM_STAGE_EMBED)) return;
  for (int l = 0; l < D.n_layers; ++l) {
    const LayerW& W = R->layers[l];
    DevBatch bl = b;  // this layer's block of the session KV pages
    if (R->kv_pool) bl.kv = R->kv_pool + (size_t)l * 2 * kPageRows * Hk * hd;
    // The last layer's prefix rows feed nothing but their K and V (read by the
    // branch tiles): after its QKV projection it runs over the branch rows
    // [0, n_brows) only -- no prefix attention, O projection, MLP.  A debug
    // stop reads whole layers, so it keeps every row.
    const bool tail = l == D.n_layers - 1 && q.stop_layer < 0;
    q.brows = false;
    q.run(DUOLM_K_RMSNORM, [&] { launch_rmsnorm(s, c.T, ln->X, W.attn_norm, ln->Xn, dT, d, eps); });
    if (q.stop(l, DUOLM_STAGE_ATTN_NORM)) return;
    q.run(DUOLM_K_GEMM_QKV,
          [&] { launch_gemm(s, EPI_BF16, c.T, ln->Xn, d, W.wqkv, d, ln->QKV, nq, dT, nq, d, c.share); });
    if (q.stop(l, DUOLM_STAGE_QKV)) return;
    q.run(DUOLM_K_QK_ROPE, [&] {
      launch_qk_rope(s, c.T, ln->QKV, nq, b.hdr, ln->pos, W.q_norm, W.k_norm, R->rope, H, Hk, hd, eps);
    });
    if (q.stop(l, DUOLM_STAGE_QK_ROPE)) return;
    if (c.session) launch_kv_store(s, c.T, ln->QKV, nq, bl, H, Hk, hd);
    // prefix and branch tiles in one launch, side by side on the chip; apart
    // when either kind is being timed
    const bool split = ((R->prof_mask >> DUOLM_K_ATTN_PREFIX) & 1u) || ((R->prof_mask >> DUOLM_K_ATTN_BRANCH) & 1u);
    if (tail) {
      if (c.bitems > 0)
        q.run(DUOLM_K_ATTN_BRANCH,
              [&] { launch_attn(s, hd, 0, c.bitems, ln->QKV, nq, ln->Ob, H * hd, bl, H, Hk, scale_log2); });
    } else if (split) {
      q.run(DUOLM_K_ATTN_PREFIX,
            [&] { launch_attn(s, hd, c.pitems, 0, ln->QKV, nq, ln->Ob, H * hd, bl, H, Hk, scale_log2); });
      if (c.bitems > 0)
        q.run(DUOLM_K_ATTN_BRANCH,
              [&] { launch_attn(s, hd, 0, c.bitems, ln->QKV, nq, ln->Ob, H * hd, bl, H, Hk, scale_log2); });
    } else {
      q.run(DUOLM_K_ATTN_PREFIX,
            [&] { launch_attn(s, hd, c.pitems, c.bitems, ln->QKV, nq, ln->Ob, H * hd, bl, H, Hk, scale_log2); });
    }
    if (q.stop(l, DUOLM_STAGE_ATTN)) return;
    const int cr = tail ? c.brows : c.T;  // rows (cap) of the rest of the layer
    const int32_t* dR = tail ? dB : dT;
    q.brows = tail;
    q.run(DUOLM_K_GEMM_O,
          [&] { launch_gemm(s, EPI_RESID, cr, ln->Ob, H * hd, W.wo, H * hd, ln->X, d, dR, d, H * hd, c.share); });
    if (q.stop(l, DUOLM_STAGE_ATTN_RESID)) return;
    q.run(DUOLM_K_RMSNORM, [&] { launch_rmsnorm(s, cr, ln->X, W.mlp_norm, ln->Xn, dR, d, eps); });
    if (q.stop(l, DUOLM_STAGE_MLP_NORM)) return;
    q.run(DUOLM_K_GEMM_GATEUP,
          [&] { launch_gemm(s, EPI_SWIGLU, cr, ln->Xn, d, W.wgu, d, ln->Hb, F, dR, 2 * F, d, c.share); });
    if (q.stop(l, DUOLM_STAGE_SWIGLU)) return;
    q.run(DUOLM_K_GEMM_DOWN,
          [&] { launch_gemm(s, EPI_RESID, cr, ln->Hb, F, W.wdown, F, ln->X, d, dR, d, F, c.share); });
    q.brows = false;
    if (q.stop(l, DUOLM_STAGE_LAYER_OUT)) return;
  }
  if (q.stop_layer >= 0) return;
  q.run(DUOLM_K_HEAD, [&] { launch_head(s, c.scores, ln->X, b, R->final_norm, R->head, scores, d, eps); });
}

// Upload one launch's descriptor block (pinned double buffer).
int upload_plan(duolm_ranker* R, Lane& Ln, const Plan& P, hipStream_t s) {
  const int slot = Ln.meta_slot;
  Ln.meta_slot ^= 1;
  HIP_TRY(hipEventSynchronize(Ln.meta_free[slot]));
  char* h = Ln.h_meta[slot];
  CallHeader hdr{};
  hdr.T = P.T;
  hdr.n_seq = (int)P.seqs.size();
  hdr.n_pitems = (int)P.pitems.size();
  hdr.n_bitems = (int)P.bitems.size();
  hdr.n_scores = (int)P.head_rows.size();
  hdr.score_off = P.score_off;
  hdr.n_inline = R->call_n_inline;
  hdr.n_brows = P.TB;
  memcpy(h, &hdr, sizeof(hdr));
  memcpy(h + Ln.off_sro, P.seq_row_off.data(), P.seq_row_off.size() * 4);
  memcpy(h + Ln.off_seq, P.seqs.data(), P.seqs.size() * sizeof(SeqDesc));
  memcpy(h + Ln.off_pi, P.pitems.data(), P.pitems.size() * sizeof(WorkItem));
  memcpy(h + Ln.off_bi, P.bitems.data(), P.bitems.size() * sizeof(WorkItem));
  memcpy(h + Ln.off_hr, P.head_rows.data(), P.head_rows.size() * 4);
  if (!P.pages.empty()) memcpy(h + Ln.off_pt, P.pages.data(), P.pages.size() * 4);
  // copy up to the end of the last used section in one transfer when the gaps
  // are small, else section by section
  const size_t end_used = P.pages.empty() ? Ln.off_hr + P.head_rows.size() * 4 : Ln.off_pt + P.pages.size() * 4;
  if (end_used <= 256 * 1024) {
    HIP_TRY(hipMemcpyAsync(Ln.d_meta, h, end_used, hipMemcpyHostToDevice, s));
  } else {
    const size_t offs[7] = {0, Ln.off_sro, Ln.off_seq, Ln.off_pi, Ln.off_bi, Ln.off_hr, Ln.off_pt};
    const size_t lens[7] = {sizeof(CallHeader), P.seq_row_off.size() * 4, P.seqs.size() * sizeof(SeqDesc),
                            P.pitems.size() * sizeof(WorkItem), P.bitems.size() * sizeof(WorkItem),
                            P.head_rows.size() * 4, P.pages.size() * 4};
    for (int i = 0; i < 7; ++i)
      if (lens[i]) HIP_TRY(hipMemcpyAsync(Ln.d_meta + offs[i], h + offs[i], lens[i], hipMemcpyHostToDevice, s));
  }
  HIP_TRY(hipEventRecord(Ln.meta_free[slot], s));
  return DUOLM_OK;
}

// A timed launch on the call's device timeline (ms after the call's
// reference event).
struct Span {
  int cls;
  double t0, t1;
};

// Read one launch's timed events: its work goes to the counters now, its
// interval to `spans` (the class's device time is settled per call).
void add_stats(duolm_ranker* R, const Plan& P, const std::vector<Timed>& timed, std::vector<Span>& spans) {
  double fl[DUOLM_K_COUNT], by[DUOLM_K_COUNT], flb[DUOLM_K_COUNT], byb[DUOLM_K_COUNT];
  launch_work(R, P, fl, by, P.T);
  launch_work(R, P, flb, byb, P.TB);
  for (const Timed& t : timed) {
    float a = 0.f, b = 0.f;
    if (hipEventElapsedTime(&a, R->call_t0, t.a) != hipSuccess ||
        hipEventElapsedTime(&b, R->call_t0, t.b) != hipSuccess)
      continue;
    duolm_kernel_stats& st = R->stats[t.cls];
    st.launches += 1;
    st.flops += (t.brows ? flb : fl)[t.cls];
    st.bytes += (t.brows ? byb : by)[t.cls];
    spans.push_back({t.cls, a, b});
  }
}

// Device time per class: the length of the union of its launches' intervals
// (the sum of their durations when they do not overlap; launches of the two
// lanes that run at the same time count once).
void settle_spans(duolm_ranker* R, std::vector<Span>& spans) {
  std::sort(spans.begin(), spans.end(), [](const Span& x, const Span& y) {
    return x.cls != y.cls ? x.cls < y.cls : x.t0 < y.t0;
  });
  for (size_t i = 0; i < spans.size();) {
    const int cls = spans[i].cls;
    double total = 0, lo = spans[i].t0, hi = spans[i].t1;
    for (; i < spans.size() && spans[i].cls == cls; ++i) {
      if (spans[i].t0 > hi) {
        total += hi - lo;
        lo = spans[i].t0;
        hi = spans[i].t1;
      } else {
        hi = std::max(hi, spans[i].t1);
      }
    }
    total += hi - lo;
    R->stats[cls].total_ms += total;
  }
  spans.clear();
}

// Run one planned launch: upload, then eager enqueue or graph replay.
int run_launch(duolm_ranker* R, Lane& Ln, const Plan& P, hipStream_t s, bool use_graph, std::vector<Timed>* timed,
               int share) {
  int rc = upload_plan(R, Ln, P, s);
  if (rc) return rc;
  if (!use_graph) {
    Caps c{P.T, (int)P.seqs.size(), (int)P.pitems.size(), (int)P.bitems.size(), (int)P.head_rows.size(),
           (int)P.pages.size(), P.session ? 1 : 0, P.TB, share};
    Enq q{R, &Ln, s, R->prof_mask ? timed : nullptr, nullptr};
    enqueue_forward(q, c);
    HIP_TRY(hipGetLastError());
    return DUOLM_OK;
  }
  Caps c{std::min(bucket(P.T), Ln.cap_T), std::min(bucket((int)P.seqs.size()), Ln.cap_seq),
         std::min(bucket((int)P.pitems.size()), Ln.cap_pi), std::min(bucket((int)P.bitems.size()), Ln.cap_bi),
         std::min(bucket((int)P.head_rows.size()), Ln.cap_hs), 0, P.session ? 1 : 0,
         std::min(bucket(P.TB), Ln.cap_T), share};
  auto it = Ln.graphs.find(c);
  if (it == Ln.graphs.end()) {
    GraphEntry ge;
    Enq q{R, &Ln, s, nullptr, &ge};
    q.note(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    if (q.cap_err == hipSuccess) enqueue_forward(q, c);
    hipGraph_t g = nullptr;
    q.note(hipStreamEndCapture(s, &g));
    if (q.cap_err == hipSuccess) q.note(hipGraphInstantiate(&ge.exec, g, nullptr, nullptr, 0));
    if (g) (void)hipGraphDestroy(g);
    if (q.cap_err != hipSuccess) {
      free_graph(ge);
      return fail(DUOLM_EHIP, "graph capture: %s", hipGetErrorString(q.cap_err));
    }
    it = Ln.graphs.emplace(c, std::move(ge)).first;
  }
  HIP_TRY(hipGraphLaunch(it->second.exec, s));
  // the graph's events hold this replay's times until its next replay: the
  // caller reads them before launching the same graph again
  if (timed) timed->insert(timed->end(), it->second.timed.begin(), it->second.timed.end());
  return DUOLM_OK;
}

struct CallInput {
  const int32_t* prefix_len;
  const int32_t* n_cand;
  const int32_t* cand_len;  // ids (rows) per candidate, per request; null: 1
  int n_req;
};

int cand_rows(const CallInput& in, int i) { return in.cand_len && in.cand_len[i] > 1 ? in.cand_len[i] : 1; }

// Longest candidate branch the attention tiles take whole.
int max_cand_len(const duolm_ranker* R) {
  return std::min(DUOLM_MAX_CAND_LEN, attn_rows_per_item(true, R->dims.n_heads / R->dims.n_kv_heads));
}

// Pinned host staging, so that host ids go up and scores come down by DMA
// straight from page-locked memory.  Calls are synchronous, so nothing is in
// flight from it when it grows.
int ensure_stage(duolm_ranker* R, size_t bytes) {
  if (bytes <= R->cap_stage) return DUOLM_OK;
  const size_t cap = std::max(bytes, R->cap_stage * 2);
  char* p = nullptr;
  if (hipHostMalloc((void**)&p, cap) != hipSuccess) return fail(DUOLM_ENOMEM, "pinned staging (%zu bytes)", cap);
  if (R->h_stage) (void)hipHostFree(R->h_stage);
  R->h_stage = p;
  R->cap_stage = cap;
  return DUOLM_OK;
}

int validate_lengths(duolm_ranker* R, const CallInput& in, int64_t& total_ids, int64_t& total_scores) {
  if (in.n_req < 1) return fail(DUOLM_EINVAL, "n_req must be >= 1");
  total_ids = 0;
  total_scores = 0;
  for (int i = 0; i < in.n_req; ++i) {
    const int L = in.prefix_len[i], K = in.n_cand[i];
    if (in.cand_len && (in.cand_len[i] < 0 || in.cand_len[i] > max_cand_len(R)))
      return fail(DUOLM_EINVAL, "request %d: cand_len %d outside [0, %d]", i, in.cand_len[i], max_cand_len(R));
    const int m = cand_rows(in, i);
    if (L < 1) return fail(DUOLM_EINVAL, "request %d: prefix_len %d < 1", i, L);
    if (K < 1) return fail(DUOLM_EINVAL, "request %d: n_cand %d < 1", i, K);
    if (L + m - 1 > R->dims.max_prefix)
      return fail(DUOLM_EINVAL, "request %d: prefix_len %d + cand_len %d over %d", i, L, m, R->dims.max_prefix + 1);
    if ((int64_t)L + (int64_t)K * m > R->max_rows)
      return fail(DUOLM_EINVAL, "request %d: L + K * cand_len = %lld over the %lld-row launch limit", i,
                  (long long)L + (long long)K * m, (long long)R->max_rows);
    total_ids += L + (int64_t)K * m;
    total_scores += K;
  }
  if (total_ids > INT32_MAX / 2) return fail(DUOLM_EINVAL, "batch too large");
  return DUOLM_OK;
}

// Split the call into launches of at most max_rows rows.
// Where a call's sequences are cut into launches: at the row limit, and --
// when the call is large enough to run as concurrent pieces, one per lane --
// at sequence boundaries near each 1/kLanes of its rows.
struct Splitter {
  duolm_ranker* R;
  int64_t total;
  int pieces, cuts = 0;
  int64_t done = 0;  // rows in the closed launches
  Splitter(duolm_ranker* r, int64_t total_rows, int64_t n_seqs, bool lanes = true)
      : R(r), total(total_rows),
        pieces(lanes && n_seqs >= 2 && total_rows >= kLaneMinRows && total_rows <= r->max_rows
                   ? (int)std::min<int64_t>(kLanes, n_seqs) : 1) {}
  // before adding a sequence of `rows` rows; score_next is its first score
  void before(std::vector<Plan>& plans, int64_t rows, int score_next) {
    const Plan& P = plans.back();
    const bool full = P.T > 0 && P.T + rows > R->max_rows;
    const bool piece = cuts + 1 < pieces && P.T > 0 && (done + P.T) * pieces >= total * (cuts + 1);
    if (!full && !piece) return;
    if (piece) ++cuts;
    done += P.T;
    plan_close(R, plans.back());
    plans.emplace_back();
    plans.back().score_off = score_next;
  }
};

void build_plans(duolm_ranker* R, const CallInput& in, int mode, std::vector<Plan>& plans, bool lanes = true) {
  plans.clear();
  plans.emplace_back();
  int64_t total = 0, n_seqs = 0;
  for (int i = 0; i < in.n_req; ++i) {
    const int64_t L = in.prefix_len[i], K = in.n_cand[i], m = cand_rows(in, i);
    total += mode == DUOLM_MODE_MIS ? L + K * m : K * (L + m);
    n_seqs += mode == DUOLM_MODE_MIS ? 1 : K;
  }
  Splitter cut(R, total, n_seqs, lanes);
  int64_t id_off = 0;
  int score = 0;
  for (int i = 0; i < in.n_req; ++i) {
    const int L = in.prefix_len[i], K = in.n_cand[i], m = cand_rows(in, i);
    if (mode == DUOLM_MODE_MIS) {
      cut.before(plans, L + (int64_t)K * m, score);
      plan_add_seq(R, plans.back(), L, K, m, (int)id_off, L, (int)(id_off + L));
    } else {
      // Each candidate appended alone to its prefix: a sequence of its own
      // with the prefix recomputed.  With one candidate the tree mask is the
      // causal mask over L + m rows, so this is the plain causal forward; its
      // m rows go through the branch tiles, the same reduction order as in
      // MIS, which keeps the two modes' scores identical.
      for (int j = 0; j < K; ++j) {
        cut.before(plans, L + m, score + j);
        plan_add_seq(R, plans.back(), L, 1, m, (int)id_off, L, (int)(id_off + L + (int64_t)j * m));
      }
    }
    score += K;
    id_off += L + (int64_t)K * m;
  }
  plan_close(R, plans.back());
}

int mode_ok(const duolm_opts* o) {
  if (o && o->mode != DUOLM_MODE_MIS && o->mode != DUOLM_MODE_INDEPENDENT) return fail(DUOLM_EINVAL, "bad mode");
  if (o && (o->max_lanes < 0 || o->max_lanes > kLanes)) return fail(DUOLM_EINVAL, "bad max_lanes %d", o->max_lanes);
  return DUOLM_OK;
}

bool lanes_allowed(const duolm_opts* o) { return !o || o->max_lanes != 1; }

// Range-check host ids while copying them into the pinned stage.
int stage_host_ids(duolm_ranker* R, const int32_t* ids, int64_t total_ids, int64_t n_inline) {
  const int64_t lim = (int64_t)R->dims.vocab + R->n_vid + n_inline;
  int32_t* st = (int32_t*)R->h_stage;
  for (int64_t i = 0; i < total_ids; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || id >= lim) {
      if (id >= R->dims.vocab && R->n_vid + n_inline == 0 && id >= 0)
        return fail(DUOLM_ESTATE, "id %d at position %lld is a VID but no item table is loaded", id, (long long)i);
      return fail(DUOLM_ERANGE, "id %d at position %lld outside [0, %lld)", id, (long long)i, (long long)lim);
    }
    st[i] = id;
  }
  return DUOLM_OK;
}

// Run planned launches: grow the buffers, upload the ids, launch every plan
// (graph or eager), check the device id flag, return the scores.  `ids` is
// the pinned stage or device memory (ids_dev).
int run_plans(duolm_ranker* R, const std::vector<Plan>& plans, const int32_t* ids, bool ids_dev, int64_t total_ids,
              float* out, bool out_dev, int64_t total_scores, hipStream_t s, bool use_graph,
              const uint16_t* inline_rows = nullptr, int64_t n_inline = 0) {
  int rc;
  // plan i runs on lane i % nl: lane 0 on the call's stream, the others on their own
  const int nl = (int)std::min<size_t>(plans.size(), kLanes);
  for (int li = 0; li < nl; ++li) {
    int maxT = 0, mseq = 0, mpi = 0, mbi = 0, mhs = 0, mpt = 0;
    for (size_t i = li; i < plans.size(); i += nl) {
      const Plan& P = plans[i];
      maxT = std::max(maxT, P.T);
      mseq = std::max(mseq, (int)P.seqs.size());
      mpi = std::max(mpi, (int)P.pitems.size());
      mbi = std::max(mbi, (int)P.bitems.size());
      mhs = std::max(mhs, (int)P.head_rows.size());
      mpt = std::max(mpt, (int)P.pages.size());
    }
    if ((rc = ensure_rows(R, R->lanes[li], maxT))) return rc;
    if ((rc = ensure_meta(R, R->lanes[li], mseq, mpi, mbi, mhs, mpt))) return rc;
  }
  if ((rc = ensure_buf(R, R->d_ids, R->cap_ids, std::max<int64_t>(1, total_ids)))) return rc;
  if ((rc = ensure_buf(R, R->d_out, R->cap_out, std::max<int64_t>(1, total_scores)))) return rc;
  if ((rc = ensure_buf(R, R->d_inline, R->cap_inline, std::max<int64_t>(1, n_inline) * R->dims.d_model))) return rc;
  if (s != R->stream) HIP_TRY(hipStreamSynchronize(R->stream));
  R->call_n_inline = (int32_t)n_inline;
  if (n_inline > 0)
    HIP_TRY(hipMemcpyAsync(R->d_inline, inline_rows, (size_t)n_inline * R->dims.d_model * 2, hipMemcpyHostToDevice, s));
  if (total_ids > 0)
    HIP_TRY(hipMemcpyAsync(R->d_ids, ids, (size_t)total_ids * 4,
                           ids_dev ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice, s));
  *R->h_err = 0;
  HIP_TRY(hipMemcpyAsync(R->d_err, R->h_err, 4, hipMemcpyHostToDevice, s));
  if (nl > 1) {  // the other lanes start once the ids and the error flag are on the device
    HIP_TRY(hipEventRecord(R->ids_ready, s));
    for (int li = 1; li < nl; ++li) HIP_TRY(hipStreamWaitEvent(R->lanes[li].stream, R->ids_ready, 0));
  }
  R->ev_used = 0;
  if (R->prof_mask) HIP_TRY(hipEventRecord(R->call_t0, s));  // the call's timeline origin (before lane 1 forks)
  std::vector<std::vector<Timed>> timed(plans.size());
  std::vector<Span> spans;
  for (size_t i = 0; i < plans.size(); ++i) {
    Lane& Ln = R->lanes[i % nl];
    hipStream_t ls = i % nl == 0 ? s : Ln.stream;
    if (R->prof_mask && i >= (size_t)nl) {
      // the lane's previous launch may have replayed the graph this one
      // replays: read its times before they are overwritten
      HIP_TRY(hipStreamSynchronize(ls));
      add_stats(R, plans[i - nl], timed[i - nl], spans);
      timed[i - nl].clear();
    }
    if ((rc = run_launch(R, Ln, plans[i], ls, use_graph, &timed[i], nl))) {
      (void)sync_all(R);
      (void)hipStreamSynchronize(s);
      return rc;
    }
  }
  for (int li = 1; li < nl; ++li) {
    HIP_TRY(hipEventRecord(R->lanes[li].done, R->lanes[li].stream));
    HIP_TRY(hipStreamWaitEvent(s, R->lanes[li].done, 0));
  }
  // The error flag and the scores go out behind the last launch, so the host
  // waits once: device scores are copied by a kernel that skips the copy when
  // the flag is set; host scores land in the pinned stage (its ids upload is
  // earlier on this stream) and reach `out` only if the flag is clear.
  HIP_TRY(hipMemcpyAsync(R->h_err, R->d_err, 4, hipMemcpyDeviceToHost, s));
  if (total_scores > 0) {
    if (out_dev) {
      launch_copy_scores(s, out, R->d_out, (int)total_scores, R->d_err);
      HIP_TRY(hipGetLastError());
    } else {
      HIP_TRY(hipMemcpyAsync(R->h_stage, R->d_out, (size_t)total_scores * 4, hipMemcpyDeviceToHost, s));
    }
  }
  HIP_TRY(hipStreamSynchronize(s));
  if (R->prof_mask) {
    for (size_t i = 0; i < plans.size(); ++i)
      if (!timed[i].empty()) add_stats(R, plans[i], timed[i], spans);
    settle_spans(R, spans);
  }
  if (*R->h_err) return fail(DUOLM_ERANGE, "an id in the device batch is outside [0, V + N)");
  if (total_scores > 0 && !out_dev) memcpy(out, R->h_stage, (size_t)total_scores * 4);
  return DUOLM_OK;
}

// Shared body of the host and device entry points.  `ids` is host memory
// when ids_dev is false.  Scores go to `out` (host or device).
int score_impl(duolm_ranker* R, const CallInput& in, const int32_t* ids, bool ids_dev, float* out, bool out_dev,
               const duolm_opts* opts, const uint16_t* inline_rows = nullptr, int64_t n_inline = 0) {
  if (!R || !in.prefix_len || !in.n_cand || !ids || !out) return fail(DUOLM_EINVAL, "NULL argument");
  int rc = mode_ok(opts);
  if (rc) return rc;
  const int mode = opts ? opts->mode : DUOLM_MODE_MIS;
  const bool use_graph = opts ? opts->use_graph != 0 : true;
  hipStream_t s = (opts && opts->hip_stream) ? (hipStream_t)opts->hip_stream : R->stream;
  int64_t total_ids = 0, total_scores = 0;
  rc = validate_lengths(R, in, total_ids, total_scores);
  if (rc) return rc;
  HIP_TRY(hipSetDevice(R->device));
  if (!ids_dev || !out_dev) {
    if ((rc = ensure_stage(R, (size_t)std::max(total_ids, total_scores) * 4))) return rc;
  }
  if (!ids_dev) {
    if ((rc = stage_host_ids(R, ids, total_ids, n_inline))) return rc;
    ids = (const int32_t*)R->h_stage;
  }
  std::vector<Plan> plans;
  build_plans(R, in, mode, plans, lanes_allowed(opts));
  return run_plans(R, plans, ids, ids_dev, total_ids, out, out_dev, total_scores, s, use_graph, inline_rows, n_inline);
}

// Concatenate host requests as [prefix_0, cands_0, prefix_1, ...].  Requests
// that ship their item vectors have each id >= V rewritten to V + N + j, row j
// of the call's inline table.
int flatten_requests(const duolm_ranker* R, const duolm_request* reqs, int n_req, std::vector<int32_t>& L,
                     std::vector<int32_t>& K, std::vector<int32_t>& M, std::vector<int32_t>& ids,
                     std::vector<uint16_t>& inl) {
  if (!reqs || n_req < 1) return fail(DUOLM_EINVAL, "need n_req >= 1 requests");
  L.resize(n_req);
  K.resize(n_req);
  M.resize(n_req);
  size_t total = 0;
  for (int i = 0; i < n_req; ++i) {
    if (reqs[i].prefix_len < 1 || reqs[i].n_cand < 1)
      return fail(DUOLM_EINVAL, "request %d: prefix_len and n_cand must be >= 1", i);
    if (!reqs[i].ids || !reqs[i].cand_ids) return fail(DUOLM_EINVAL, "request %d: NULL ids", i);
    if (reqs[i].cand_len < 0 || reqs[i].cand_len > max_cand_len(R))
      return fail(DUOLM_EINVAL, "request %d: cand_len %d outside [0, %d]", i, reqs[i].cand_len, max_cand_len(R));
    L[i] = reqs[i].prefix_len;
    K[i] = reqs[i].n_cand;
    M[i] = reqs[i].cand_len > 1 ? reqs[i].cand_len : 1;
    total += (size_t)L[i] + (size_t)K[i] * M[i];
  }
  ids.resize(total);
  inl.clear();
  const int V = R->dims.vocab, d = R->dims.d_model;
  int64_t n_inl = 0;
  size_t o = 0;
  for (int i = 0; i < n_req; ++i) {
    const size_t start = o;
    memcpy(&ids[o], reqs[i].ids, (size_t)L[i] * 4);
    o += L[i];
    memcpy(&ids[o], reqs[i].cand_ids, (size_t)K[i] * M[i] * 4);
    o += (size_t)K[i] * M[i];
    if (!reqs[i].inline_vecs) {
      const int64_t lim = (int64_t)V + R->n_vid;
      for (size_t t = start; t < o; ++t) {
        const int32_t id = ids[t];
        if (id >= V && R->n_vid == 0)
          return fail(DUOLM_ESTATE, "request %d: id %d is a VID but no item table is loaded", i, id);
        if (id < 0 || id >= lim)
          return fail(DUOLM_ERANGE, "request %d: id %d outside [0, %lld)", i, id, (long long)lim);
      }
    } else {
      int64_t j = 0;
      for (size_t t = start; t < o; ++t) {
        if (ids[t] < 0) return fail(DUOLM_ERANGE, "request %d: negative id %d", i, ids[t]);
        if (ids[t] >= V) {
          ids[t] = (int32_t)(V + R->n_vid + n_inl + j);
          ++j;
        }
      }
      if ((int64_t)V + R->n_vid + n_inl + j > INT32_MAX) return fail(DUOLM_EINVAL, "too many inline vectors");
      inl.insert(inl.end(), reqs[i].inline_vecs, reqs[i].inline_vecs + j * d);
      n_inl += j;
    }
  }
  return DUOLM_OK;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

int duolm_load_ranker(const char* path, int hip_device, duolm_ranker** out) {
  if (!path || !out) return fail(DUOLM_EINVAL, "NULL argument");
  const int fd = open(path, O_RDONLY);
  if (fd < 0) return fail(DUOLM_EIO, "cannot open %s", path);
  struct stat st;
  if (fstat(fd, &st) != 0 || st.st_size < 64) {
    close(fd);
    return fail(DUOLM_EIO, "cannot stat %s or file too short", path);
  }
  void* m = mmap(nullptr, (size_t)st.st_size, PROT_READ, MAP_PRIVATE, fd, 0);
  close(fd);
  if (m == MAP_FAILED) return fail(DUOLM_EIO, "cannot map %s", path);
  const int rc = create_from_blob(m, (uint64_t)st.st_size, hip_device, out);
  munmap(m, (size_t)st.st_size);
  return rc;
}

int duolm_load_ranker_mem(const void* blob, uint64_t nbytes, int hip_device, duolm_ranker** out) {
  return create_from_blob(blob, nbytes, hip_device, out);
}

int duolm_load_vid_table(duolm_ranker* R, const uint16_t* rows, int64_t n_rows) {
  if (!R || !rows) return fail(DUOLM_EINVAL, "NULL argument");
  if (n_rows < 1) return fail(DUOLM_EINVAL, "n_rows must be >= 1");
  if ((int64_t)R->dims.vocab + n_rows > INT32_MAX) return fail(DUOLM_EINVAL, "V + n_rows exceeds int32 ids");
  HIP_TRY(hipSetDevice(R->device));
  HIP_TRY(hipStreamSynchronize(R->stream));
  const size_t bytes = (size_t)n_rows * R->dims.d_model * 2;
  uint16_t* p = nullptr;
  if (hipMalloc((void**)&p, bytes) != hipSuccess) return fail(DUOLM_ENOMEM, "item table (%zu bytes)", bytes);
  if (hipMemcpy(p, rows, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(p);
    return fail(DUOLM_EHIP, "item table upload failed");
  }
  if (R->vid) (void)hipFree(R->vid);
  R->vid = p;
  R->n_vid = n_rows;
  R->dims.n_vid = n_rows;
  drop_graphs(R);  // graphs bake the table pointer and size
  return DUOLM_OK;
}

// ---------------------------------------------------------------------------
// offline export of item vectors (the step before the table is served)
// ---------------------------------------------------------------------------
namespace {

// p must be device memory of `device` holding [p, p + bytes) inside one
// allocation; a host or foreign pointer would fault the kernel instead
int check_dev_range(const void* p, size_t bytes, int device, const char* what) {
  if (!p) return fail(DUOLM_EINVAL, "%s is NULL", what);
  if ((uintptr_t)p % 16) return fail(DUOLM_EINVAL, "%s is not 16-byte aligned", what);
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess || at.type != hipMemoryTypeDevice) {
    (void)hipGetLastError();
    return fail(DUOLM_EINVAL, "%s is not device memory", what);
  }
  if (at.device != device) return fail(DUOLM_EINVAL, "%s lives on device %d, not %d", what, at.device, device);
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(DUOLM_EINVAL, "%s: allocation range unknown", what);
  }
  if ((const char*)p + bytes > (const char*)base + size)
    return fail(DUOLM_EINVAL, "%s: %zu bytes do not fit its allocation", what, bytes);
  return DUOLM_OK;
}

size_t dtype_bytes(int32_t dt) { return dt == DUOLM_DTYPE_F32 ? 4 : 2; }

int check_export_args(int32_t dt, int64_t n_rows, int32_t d, double rho, double gamma, double eps) {
  if (dt != DUOLM_DTYPE_F32 && dt != DUOLM_DTYPE_BF16 && dt != DUOLM_DTYPE_F16)
    return fail(DUOLM_EINVAL, "bad input dtype %d", dt);
  if (n_rows < 0 || n_rows > INT32_MAX) return fail(DUOLM_EINVAL, "n_rows %lld out of range", (long long)n_rows);
  if (d < 8 || d % 8 || d > DUOLM_MAX_EXPORT_DIM)
    return fail(DUOLM_EINVAL, "d = %d: must be a multiple of 8 in [8, %d]", d, DUOLM_MAX_EXPORT_DIM);
  if (!std::isfinite(rho) || !std::isfinite(gamma) || !(eps >= 0.0) || !std::isfinite(eps))
    return fail(DUOLM_EINVAL, "rho and gamma must be finite and eps finite and >= 0");
  if (!std::isfinite(rho * std::exp(gamma))) return fail(DUOLM_EINVAL, "rho * e^gamma overflows");
  return DUOLM_OK;
}

}  // namespace

int duolm_export_item_vectors(const void* d_a, int32_t a_dtype, int64_t n_rows, int32_t d, double rho,
                              double gamma, double eps, uint16_t* d_z, void* hip_stream) {
  int rc = check_export_args(a_dtype, n_rows, d, rho, gamma, eps);
  if (rc) return rc;
  if (n_rows == 0) return DUOLM_OK;
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if ((rc = check_dev_range(d_a, (size_t)n_rows * d * dtype_bytes(a_dtype), dev, "d_a"))) return rc;
  if ((rc = check_dev_range(d_z, (size_t)n_rows * d * 2, dev, "d_z"))) return rc;
  if (!launch_export((hipStream_t)hip_stream, a_dtype, d_a, n_rows, d, rho * std::exp(gamma), eps, d_z))
    return fail(DUOLM_EINVAL, "unsupported export shape");
  HIP_TRY(hipGetLastError());
  return DUOLM_OK;
}

int duolm_export_vid_table(duolm_ranker* R, const void* d_a, int32_t a_dtype, int64_t n_rows, double rho,
                           double gamma, double eps) {
  if (!R) return fail(DUOLM_EINVAL, "NULL argument");
  const int d = R->dims.d_model;
  int rc = check_export_args(a_dtype, n_rows, d, rho, gamma, eps);
  if (rc) return rc;
  if (n_rows < 1) return fail(DUOLM_EINVAL, "n_rows must be >= 1");
  if ((int64_t)R->dims.vocab + n_rows > INT32_MAX) return fail(DUOLM_EINVAL, "V + n_rows exceeds int32 ids");
  HIP_TRY(hipSetDevice(R->device));
  if ((rc = check_dev_range(d_a, (size_t)n_rows * d * dtype_bytes(a_dtype), R->device, "d_a"))) return rc;
  HIP_TRY(hipStreamSynchronize(R->stream));
  const size_t bytes = (size_t)n_rows * d * 2;
  uint16_t* p = nullptr;
  if (hipMalloc((void**)&p, bytes) != hipSuccess) return fail(DUOLM_ENOMEM, "item table (%zu bytes)", bytes);
  const bool ok = launch_export(R->stream, a_dtype, d_a, n_rows, d, rho * std::exp(gamma), eps, p);
  const hipError_t e1 = hipGetLastError();
  const hipError_t e2 = hipStreamSynchronize(R->stream);
  if (!ok || e1 != hipSuccess || e2 != hipSuccess) {
    (void)hipFree(p);
    return fail(DUOLM_EHIP, "item export failed: %s", hipGetErrorString(e1 != hipSuccess ? e1 : e2));
  }
  if (R->vid) (void)hipFree(R->vid);
  R->vid = p;
  R->n_vid = n_rows;
  R->dims.n_vid = n_rows;
  drop_graphs(R);  // graphs bake the table pointer and size
  return DUOLM_OK;
}

int duolm_reference_scale(duolm_ranker* R, double* rho) {
  if (!R || !rho) return fail(DUOLM_EINVAL, "NULL argument");
  HIP_TRY(hipSetDevice(R->device));
  double* buf = nullptr;
  if (hipMalloc((void**)&buf, (kScaleBlocks + 1) * sizeof(double)) != hipSuccess)
    return fail(DUOLM_ENOMEM, "reference-scale scratch");
  launch_reference_scale(R->stream, R->embed, (int64_t)R->dims.vocab * R->dims.d_model, buf, buf + kScaleBlocks);
  double h = 0.0;
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpyAsync(&h, buf + kScaleBlocks, sizeof(double), hipMemcpyDeviceToHost, R->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(R->stream);
  (void)hipFree(buf);
  if (e != hipSuccess) return fail(DUOLM_EHIP, "reference scale: %s", hipGetErrorString(e));
  *rho = h;
  return DUOLM_OK;
}

// ---------------------------------------------------------------------------
// host input packer
// ---------------------------------------------------------------------------
namespace {

int64_t history_prefix_len(const duolm_template& t, const duolm_history& h) {
  const int64_t per_item_vids = h.item_len > 1 ? h.item_len : 1;
  return (int64_t)t.n_instruction + (int64_t)h.n_items * (1 + per_item_vids) +
         (h.n_items > 0 ? (int64_t)h.feedback_off[h.n_items] : 0) + t.n_cand_header;
}

int check_history(const duolm_template& t, const duolm_history& h, int i) {
  if (h.n_items < 0) return fail(DUOLM_EINVAL, "request %d: n_items < 0", i);
  if (h.item_len < 0 || h.item_len > DUOLM_MAX_CAND_LEN)
    return fail(DUOLM_EINVAL, "request %d: item_len %d outside [0, %d]", i, h.item_len, DUOLM_MAX_CAND_LEN);
  if (h.cand_len < 0 || h.cand_len > DUOLM_MAX_CAND_LEN)
    return fail(DUOLM_EINVAL, "request %d: cand_len %d outside [0, %d]", i, h.cand_len, DUOLM_MAX_CAND_LEN);
  if (h.n_cand < 1) return fail(DUOLM_EINVAL, "request %d: n_cand must be >= 1", i);
  if (!h.cand_vids) return fail(DUOLM_EINVAL, "request %d: NULL cand_vids", i);
  if (h.n_items > 0) {
    if (!h.item_vids || !h.feedback_off) return fail(DUOLM_EINVAL, "request %d: NULL item arrays", i);
    if (h.feedback_off[0] != 0) return fail(DUOLM_EINVAL, "request %d: feedback_off[0] != 0", i);
    for (int j = 0; j < h.n_items; ++j)
      if (h.feedback_off[j + 1] < h.feedback_off[j])
        return fail(DUOLM_EINVAL, "request %d: feedback_off decreases at item %d", i, j);
    if (h.feedback_off[h.n_items] > 0 && !h.feedback) return fail(DUOLM_EINVAL, "request %d: NULL feedback", i);
  }
  const int64_t L = history_prefix_len(t, h);
  if (L < 1) return fail(DUOLM_EINVAL, "request %d: empty prefix", i);
  if (L > INT32_MAX / 2) return fail(DUOLM_EINVAL, "request %d: prefix too long", i);
  return DUOLM_OK;
}

// instruction, (marker, item VIDs, feedback) per item, header, candidates
void assemble_one(const duolm_template& t, const duolm_history& h, int32_t* o) {
  const int m_item = h.item_len > 1 ? h.item_len : 1, m_cand = h.cand_len > 1 ? h.cand_len : 1;
  if (t.n_instruction) memcpy(o, t.instruction, (size_t)t.n_instruction * 4);
  o += t.n_instruction;
  for (int j = 0; j < h.n_items; ++j) {
    *o++ = t.marker;
    memcpy(o, h.item_vids + (size_t)j * m_item, (size_t)m_item * 4);
    o += m_item;
    const int32_t f0 = h.feedback_off[j], f1 = h.feedback_off[j + 1];
    if (f1 > f0) memcpy(o, h.feedback + f0, (size_t)(f1 - f0) * 4);
    o += f1 - f0;
  }
  if (t.n_cand_header) memcpy(o, t.cand_header, (size_t)t.n_cand_header * 4);
  o += t.n_cand_header;
  memcpy(o, h.cand_vids, (size_t)h.n_cand * m_cand * 4);
}

int check_template(const duolm_template* t) {
  if (!t) return fail(DUOLM_EINVAL, "NULL template");
  if (t->n_instruction < 0 || t->n_cand_header < 0) return fail(DUOLM_EINVAL, "negative template length");
  if ((t->n_instruction && !t->instruction) || (t->n_cand_header && !t->cand_header))
    return fail(DUOLM_EINVAL, "NULL template array");
  return DUOLM_OK;
}

}  // namespace

int duolm_packed_size(const duolm_template* t, const duolm_history* reqs, int32_t n_req, int64_t* n_ids) {
  if (!reqs || !n_ids || n_req < 1) return fail(DUOLM_EINVAL, "NULL argument or n_req < 1");
  int rc = check_template(t);
  if (rc) return rc;
  int64_t total = 0;
  for (int i = 0; i < n_req; ++i) {
    if ((rc = check_history(*t, reqs[i], i))) return rc;
    total += history_prefix_len(*t, reqs[i]) + (int64_t)reqs[i].n_cand * std::max(reqs[i].cand_len, 1);
  }
  *n_ids = total;
  return DUOLM_OK;
}

int duolm_pack_requests(const duolm_template* t, const duolm_history* reqs, int32_t n_req, int32_t n_threads,
                        int32_t* ids, int64_t ids_cap, int32_t* prefix_len, int32_t* n_cand, int32_t* cand_len) {
  if (!ids || !prefix_len || !n_cand || !cand_len) return fail(DUOLM_EINVAL, "NULL output");
  if (n_threads < 0) return fail(DUOLM_EINVAL, "n_threads < 0");
  int64_t total = 0;
  int rc = duolm_packed_size(t, reqs, n_req, &total);
  if (rc) return rc;
  if (total > ids_cap) return fail(DUOLM_EINVAL, "ids_cap %lld < %lld ids needed", (long long)ids_cap, (long long)total);
  // offsets first (one cheap pass), then the copies, split into contiguous
  // request ranges across threads; every range writes only its own slots
  std::vector<int64_t> off((size_t)n_req + 1, 0);
  for (int i = 0; i < n_req; ++i)
    off[i + 1] = off[i] + history_prefix_len(*t, reqs[i]) + (int64_t)reqs[i].n_cand * std::max(reqs[i].cand_len, 1);
  auto work = [&](int lo, int hi) {
    for (int i = lo; i < hi; ++i) {
      assemble_one(*t, reqs[i], ids + off[i]);
      prefix_len[i] = (int32_t)history_prefix_len(*t, reqs[i]);
      n_cand[i] = reqs[i].n_cand;
      cand_len[i] = std::max(reqs[i].cand_len, 1);
    }
  };
  // a thread costs tens of microseconds to start, about what copying 64k ids
  // takes: never more threads than 64k-id shares of the work
  const int by_work = (int)std::min<int64_t>(64, total / 65536 + 1);
  const int nt = std::min({std::max(n_threads, 1), (int)n_req, by_work});
  if (nt == 1) {
    work(0, n_req);
    return DUOLM_OK;
  }
  // balance by ids, not by request count
  std::vector<int> cut((size_t)nt + 1, n_req);
  cut[0] = 0;
  for (int k = 1, i = 0; k < nt; ++k) {
    const int64_t goal = total * k / nt;
    while (i < n_req && off[i] < goal) ++i;
    cut[k] = std::max(i, cut[k - 1]);
  }
  std::vector<std::thread> th;
  th.reserve(nt - 1);
  for (int k = 1; k < nt; ++k) th.emplace_back(work, cut[k], cut[k + 1]);
  work(cut[0], cut[1]);
  for (auto& x : th) x.join();
  return DUOLM_OK;
}

int duolm_score_packed(duolm_ranker* R, const int32_t* prefix_len, const int32_t* n_cand, const int32_t* cand_len,
                       int32_t n_req, const int32_t* ids, float* scores, const duolm_opts* opts) {
  if (!R || !prefix_len || !n_cand || !ids || !scores) return fail(DUOLM_EINVAL, "NULL argument");
  CallInput in{prefix_len, n_cand, cand_len, n_req};
  return score_impl(R, in, ids, false, scores, false, opts);
}

// ---------------------------------------------------------------------------
// sessions: prefix KV kept across calls
// ---------------------------------------------------------------------------
int duolm_kv_pool_init(duolm_ranker* R, int64_t max_rows) {
  if (!R) return fail(DUOLM_EINVAL, "NULL argument");
  if (max_rows < 1) return fail(DUOLM_EINVAL, "max_rows must be >= 1");
  if (!R->sessions.empty()) return fail(DUOLM_ESTATE, "sessions still hold pages of the current pool");
  const auto& D = R->dims;
  const int64_t n_pages = (max_rows + kPageRows - 1) / kPageRows;
  if (n_pages > INT32_MAX) return fail(DUOLM_EINVAL, "max_rows too large");
  const int64_t page_elems = (int64_t)D.n_layers * 2 * kPageRows * D.n_kv_heads * D.head_dim;
  HIP_TRY(hipSetDevice(R->device));
  HIP_TRY(hipStreamSynchronize(R->stream));
  uint16_t* p = nullptr;
  const size_t bytes = (size_t)n_pages * page_elems * 2;
  if (hipMalloc((void**)&p, bytes) != hipSuccess) return fail(DUOLM_ENOMEM, "KV pool (%zu bytes)", bytes);
  if (R->kv_pool) (void)hipFree(R->kv_pool);
  drop_graphs(R);  // graphs bake the pool address
  R->kv_pool = p;
  R->kv_pages = n_pages;
  R->page_elems = page_elems;
  R->kv_free.resize((size_t)n_pages);
  for (int64_t i = 0; i < n_pages; ++i) R->kv_free[(size_t)i] = (int32_t)(n_pages - 1 - i);
  return DUOLM_OK;
}

int duolm_kv_pool_free_pages(const duolm_ranker* R, int64_t* n_free) {
  if (!R || !n_free) return fail(DUOLM_EINVAL, "NULL argument");
  *n_free = (int64_t)R->kv_free.size();
  return DUOLM_OK;
}

int duolm_session_create(duolm_ranker* R, duolm_session** out) {
  if (!R || !out) return fail(DUOLM_EINVAL, "NULL argument");
  if (!R->kv_pool) return fail(DUOLM_ESTATE, "no KV pool: call duolm_kv_pool_init first");
  duolm_session* S = new duolm_session{R, 0, {}};
  R->sessions.insert(S);
  *out = S;
  return DUOLM_OK;
}

int duolm_session_length(const duolm_session* S, int32_t* L) {
  if (!S || !L) return fail(DUOLM_EINVAL, "NULL argument");
  *L = S->L;
  return DUOLM_OK;
}

void duolm_session_free(duolm_session* S) {
  if (!S) return;
  duolm_ranker* R = S->owner;
  R->kv_free.insert(R->kv_free.end(), S->pages.rbegin(), S->pages.rend());
  R->sessions.erase(S);
  delete S;
}

int duolm_session_step(duolm_ranker* R, duolm_session* const* sess, int32_t n, const int32_t* n_new,
                       const int32_t* n_cand, const int32_t* cand_len, const int32_t* ids, float* scores,
                       const duolm_opts* opts) {
  if (!R || !sess || !n_new || !n_cand || n < 1) return fail(DUOLM_EINVAL, "NULL argument or n < 1");
  if (opts && opts->mode != DUOLM_MODE_MIS) return fail(DUOLM_EINVAL, "sessions score in MIS mode only");
  int rc0 = mode_ok(opts);
  if (rc0) return rc0;
  const bool use_graph = opts ? opts->use_graph != 0 : true;
  hipStream_t s = (opts && opts->hip_stream) ? (hipStream_t)opts->hip_stream : R->stream;
  // validate everything before touching any session
  std::set<const duolm_session*> seen;
  int64_t total_ids = 0, total_scores = 0, need_pages = 0;
  for (int i = 0; i < n; ++i) {
    const duolm_session* S = sess[i];
    if (!S || S->owner != R) return fail(DUOLM_EINVAL, "session %d is NULL or belongs to another ranker", i);
    if (!seen.insert(S).second) return fail(DUOLM_EINVAL, "session %d appears twice", i);
    if (n_new[i] < 0 || n_cand[i] < 0) return fail(DUOLM_EINVAL, "session %d: negative count", i);
    if (cand_len && (cand_len[i] < 0 || cand_len[i] > max_cand_len(R)))
      return fail(DUOLM_EINVAL, "session %d: cand_len %d outside [0, %d]", i, cand_len[i], max_cand_len(R));
    const int m = cand_len && cand_len[i] > 1 ? cand_len[i] : 1;
    const int64_t L = (int64_t)S->L + n_new[i];
    if (n_cand[i] > 0 && L < 1) return fail(DUOLM_EINVAL, "session %d: candidates need a prefix", i);
    if (L + m - 1 > R->dims.max_prefix)
      return fail(DUOLM_EINVAL, "session %d: prefix %lld + cand_len %d over %d", i, (long long)L, m,
                  R->dims.max_prefix + 1);
    const int64_t rows = (int64_t)n_new[i] + (int64_t)n_cand[i] * m;
    if (rows > R->max_rows)
      return fail(DUOLM_EINVAL, "session %d: %lld rows over the %lld-row launch limit", i, (long long)rows,
                  (long long)R->max_rows);
    need_pages += std::max<int64_t>(0, (L + kPageRows - 1) / kPageRows - (int64_t)S->pages.size());
    total_ids += rows;
    total_scores += n_cand[i];
  }
  if (total_ids < 1) return fail(DUOLM_EINVAL, "nothing to compute");
  if (total_ids > INT32_MAX / 2) return fail(DUOLM_EINVAL, "batch too large");
  if (!ids || (total_scores > 0 && !scores)) return fail(DUOLM_EINVAL, "NULL ids or scores");
  if (need_pages > (int64_t)R->kv_free.size())
    return fail(DUOLM_ENOMEM, "KV pool: %lld pages needed, %lld free", (long long)need_pages,
                (long long)R->kv_free.size());
  HIP_TRY(hipSetDevice(R->device));
  int rc = ensure_stage(R, (size_t)std::max(total_ids, total_scores) * 4);
  if (rc) return rc;
  if ((rc = stage_host_ids(R, ids, total_ids, 0))) return rc;
  // pages for the new rows (a session keeps them if the call fails later:
  // they lie past its length and the next append writes them again)
  for (int i = 0; i < n; ++i) {
    duolm_session* S = sess[i];
    const int64_t want = ((int64_t)S->L + n_new[i] + kPageRows - 1) / kPageRows;
    while ((int64_t)S->pages.size() < want) {
      S->pages.push_back(R->kv_free.back());
      R->kv_free.pop_back();
    }
  }
  std::vector<Plan> plans(1);
  int64_t off = 0, n_seqs = 0;
  for (int i = 0; i < n; ++i) n_seqs += n_new[i] + n_cand[i] > 0;
  Splitter cut(R, total_ids, n_seqs, lanes_allowed(opts));
  int score = 0;
  for (int i = 0; i < n; ++i) {
    const duolm_session* S = sess[i];
    const int m = cand_len && cand_len[i] > 1 ? cand_len[i] : 1;
    const int rows = n_new[i] + n_cand[i] * m;
    if (rows == 0) continue;
    cut.before(plans, rows, score);
    plan_add_session(R, plans.back(), S->L, S->L + n_new[i], n_cand[i], m, (int)off, (int)(off + n_new[i]),
                     S->pages);
    off += rows;
    score += n_cand[i];
  }
  plan_close(R, plans.back());
  rc = run_plans(R, plans, (const int32_t*)R->h_stage, false, total_ids, scores, false, total_scores, s, use_graph);
  if (rc) return rc;
  for (int i = 0; i < n; ++i) sess[i]->L += n_new[i];
  return DUOLM_OK;
}

int duolm_get_dims(const duolm_ranker* R, duolm_dims* out) {
  if (!R || !out) return fail(DUOLM_EINVAL, "NULL argument");
  *out = R->dims;
  return DUOLM_OK;
}

int duolm_score_batch(duolm_ranker* R, const duolm_request* reqs, int32_t n_req, float* scores,
                      const duolm_opts* opts) {
  if (!R || !scores) return fail(DUOLM_EINVAL, "NULL argument");
  std::vector<int32_t> L, K, M, ids;
  std::vector<uint16_t> inl;
  int rc = flatten_requests(R, reqs, n_req, L, K, M, ids, inl);
  if (rc) return rc;
  CallInput in{L.data(), K.data(), M.data(), n_req};
  return score_impl(R, in, ids.data(), false, scores, false, opts, inl.data(),
                    (int64_t)(inl.size() / R->dims.d_model));
}

int duolm_score_batch_dev(duolm_ranker* R, const int32_t* prefix_len, const int32_t* n_cand,
                          const int32_t* cand_len, int32_t n_req, const int32_t* d_ids, float* d_scores,
                          const duolm_opts* opts) {
  CallInput in{prefix_len, n_cand, cand_len, n_req};
  return score_impl(R, in, d_ids, true, d_scores, true, opts);
}

int duolm_score_batch_dev_noalloc(duolm_ranker* R, const int32_t* prefix_len, const int32_t* n_cand,
                                  const int32_t* cand_len, int32_t n_req, const int32_t* d_ids, float* d_scores,
                                  const duolm_opts* opts) {
  if (!R || !prefix_len || !n_cand || !d_ids || !d_scores) return fail(DUOLM_EINVAL, "NULL argument");
  int rc = mode_ok(opts);
  if (rc) return rc;
  const int mode = opts ? opts->mode : DUOLM_MODE_MIS;
  hipStream_t s = (opts && opts->hip_stream) ? (hipStream_t)opts->hip_stream : R->stream;
  CallInput in{prefix_len, n_cand, cand_len, n_req};
  int64_t total_ids = 0, total_scores = 0;
  if ((rc = validate_lengths(R, in, total_ids, total_scores))) return rc;
  char* scr = R->device < kMaxDevices ? (char*)g_scratch_ptr[R->device] : nullptr;
  if (!scr) return fail(DUOLM_ESTATE, "no scratch on device %d", R->device);
  std::vector<Plan> plans;
  build_plans(R, in, mode, plans, false);
  if (plans.size() != 1)
    return fail(DUOLM_EINVAL, "the call needs %zu launches; the no-allocation entry point runs one", plans.size());
  const Plan& P = plans[0];
  // carve the call's buffers from the scratch: descriptor block, scores, then
  // the activations of exactly P.T rows
  Lane& Ln = R->na;
  auto a = [](size_t x) { return align_up(x, 256); };
  size_t off = a(sizeof(CallHeader));
  Ln.off_sro = off; off = a(off + (2 * P.seqs.size() + 1) * 4);
  Ln.off_seq = off; off = a(off + P.seqs.size() * sizeof(SeqDesc));
  Ln.off_pi = off; off = a(off + P.pitems.size() * sizeof(WorkItem));
  Ln.off_bi = off; off = a(off + P.bitems.size() * sizeof(WorkItem));
  Ln.off_hr = off; off = a(off + P.head_rows.size() * 4);
  Ln.off_pt = off;
  Ln.meta_bytes = off;
  if (off > kScratchMetaBytes)
    return fail(DUOLM_EINVAL, "descriptor of %zu bytes over the no-allocation limit of %zu", off, kScratchMetaBytes);
  const auto& D = R->dims;
  const size_t T = (size_t)P.T;
  const size_t bX = a(T * D.d_model * 4), bXn = a(T * D.d_model * 2), bQ = a(T * R->nqkv * 2),
               bO = a(T * D.n_heads * D.head_dim * 2), bH = a(T * D.d_ffn * 2), bP = a(T * 4),
               bS = a((size_t)total_scores * 4);
  const size_t need = kScratchMetaBytes + bS + bX + bXn + bQ + bO + bH + bP;
  if (need > kScratchBytes)
    return fail(DUOLM_EINVAL, "%zu rows need %zu bytes of scratch; the no-allocation entry point holds %zu "
                "(about %zu rows of this model)", T, need, kScratchBytes,
                (kScratchBytes - kScratchMetaBytes) / (size_t)(D.d_model * 6 + R->nqkv * 2 + D.n_heads * D.head_dim * 2 +
                                                              D.d_ffn * 2 + 8));
  HIP_TRY(hipSetDevice(R->device));
  char* p = scr;
  Ln.d_meta = p; p += kScratchMetaBytes;
  float* out = (float*)p; p += bS;
  Ln.X = (float*)p; p += bX;
  Ln.Xn = (uint16_t*)p; p += bXn;
  Ln.QKV = (uint16_t*)p; p += bQ;
  Ln.Ob = (uint16_t*)p; p += bO;
  Ln.Hb = (uint16_t*)p; p += bH;
  Ln.pos = (int32_t*)p;
  Ln.cap_T = P.T;
  if (s != R->stream) HIP_TRY(hipStreamSynchronize(R->stream));
  R->call_n_inline = 0;
  launch_fill_i32(s, R->d_err, 1, 0);
  if ((rc = upload_plan(R, Ln, P, s))) return rc;
  Caps c{P.T, (int)P.seqs.size(), (int)P.pitems.size(), (int)P.bitems.size(), (int)P.head_rows.size(),
         0, 0, P.TB, 1};
  Enq q{R, &Ln, s, nullptr, nullptr};
  q.ids = d_ids;
  q.out = out;
  enqueue_forward(q, c);
  HIP_TRY(hipGetLastError());
  HIP_TRY(hipMemcpyAsync(R->h_err, R->d_err, 4, hipMemcpyDeviceToHost, s));
  launch_copy_scores(s, d_scores, out, (int)total_scores, R->d_err);  // skipped on device when the flag is set
  HIP_TRY(hipGetLastError());
  HIP_TRY(hipStreamSynchronize(s));
  if (*R->h_err) return fail(DUOLM_ERANGE, "an id in the device batch is outside [0, V + N)");
  return DUOLM_OK;
}

int duolm_set_profiling(duolm_ranker* R, uint32_t mask) {
  if (!R) return fail(DUOLM_EINVAL, "NULL argument");
  if (mask != R->prof_mask) drop_graphs(R);  // captured graphs carry their timing events
  R->prof_mask = mask & ((1u << DUOLM_K_COUNT) - 1);
  for (auto& st : R->stats) st = duolm_kernel_stats{};
  return DUOLM_OK;
}

int duolm_get_kernel_stats(duolm_ranker* R, int32_t cls, duolm_kernel_stats* out) {
  if (!R || !out) return fail(DUOLM_EINVAL, "NULL argument");
  if (cls < 0 || cls >= DUOLM_K_COUNT) return fail(DUOLM_EINVAL, "bad kernel class %d", cls);
  *out = R->stats[cls];
  return DUOLM_OK;
}

const char* duolm_last_error(void) { return g_err.c_str(); }

void duolm_free_ranker(duolm_ranker* R) {
  if (!R) return;
  (void)hipSetDevice(R->device);
  if (R->stream) (void)hipStreamSynchronize(R->stream);
  for (Lane& Ln : R->lanes)
    if (Ln.stream) (void)hipStreamSynchronize(Ln.stream);
  drop_graphs(R);
  for (hipEvent_t e : R->ev_pool) (void)hipEventDestroy(e);
  if (R->ids_ready) (void)hipEventDestroy(R->ids_ready);
  if (R->call_t0) (void)hipEventDestroy(R->call_t0);
  for (Lane& Ln : R->lanes) {
    for (hipEvent_t e : Ln.meta_free)
      if (e) (void)hipEventDestroy(e);
    if (Ln.done) (void)hipEventDestroy(Ln.done);
    if (Ln.ws) (void)hipFree(Ln.ws);
    if (Ln.d_meta) (void)hipFree(Ln.d_meta);
    for (char* h : Ln.h_meta)
      if (h) (void)hipHostFree(h);
    if (Ln.stream) (void)hipStreamDestroy(Ln.stream);
  }
  for (hipEvent_t e : R->na.meta_free)
    if (e) (void)hipEventDestroy(e);
  for (char* h : R->na.h_meta)
    if (h) (void)hipHostFree(h);  // the na lane's device buffers are the scratch: never freed
  if (R->wblob) (void)hipFree(R->wblob);
  if (R->vid) (void)hipFree(R->vid);
  if (R->d_ids) (void)hipFree(R->d_ids);
  if (R->d_out) (void)hipFree(R->d_out);
  if (R->d_inline) (void)hipFree(R->d_inline);
  if (R->d_err) (void)hipFree(R->d_err);
  if (R->h_err) (void)hipHostFree(R->h_err);
  if (R->h_stage) (void)hipHostFree(R->h_stage);
  for (duolm_session* S : R->sessions) delete S;
  if (R->kv_pool) (void)hipFree(R->kv_pool);
  if (R->stream) (void)hipStreamDestroy(R->stream);
  delete R;
}

// ---------------------------------------------------------------------------
// test support (duolm_debug.h)
// ---------------------------------------------------------------------------
int duolm_debug_forward(duolm_ranker* R, const duolm_request* reqs, int32_t n_req, int32_t mode, int32_t layer,
                        int32_t stage, void* host_out, uint64_t nbytes) {
  if (!R || !host_out) return fail(DUOLM_EINVAL, "NULL argument");
  if (mode != DUOLM_MODE_MIS && mode != DUOLM_MODE_INDEPENDENT) return fail(DUOLM_EINVAL, "bad mode");
  if (layer < 0 || layer > R->dims.n_layers || stage < 0 || stage > DUOLM_STAGE_EMBED)
    return fail(DUOLM_EINVAL, "bad layer/stage");
  if (layer == R->dims.n_layers && stage != DUOLM_STAGE_LAYER_OUT) return fail(DUOLM_EINVAL, "bad stage");
  if (stage == DUOLM_STAGE_EMBED && layer != 0) return fail(DUOLM_EINVAL, "embed stage is layer 0 only");
  std::vector<int32_t> L, K, M, ids;
  std::vector<uint16_t> inl;
  int rc = flatten_requests(R, reqs, n_req, L, K, M, ids, inl);
  if (rc) return rc;
  if (!inl.empty()) return fail(DUOLM_EINVAL, "debug forward takes table ids only");
  CallInput in{L.data(), K.data(), M.data(), n_req};
  int64_t total_ids = 0, total_scores = 0;
  if ((rc = validate_lengths(R, in, total_ids, total_scores))) return rc;
  const int64_t lim = (int64_t)R->dims.vocab + R->n_vid;
  for (int32_t id : ids)
    if (id < 0 || id >= lim) return fail(DUOLM_ERANGE, "id %d outside [0, %lld)", id, (long long)lim);
  std::vector<Plan> plans;
  build_plans(R, in, mode, plans, false);
  if (plans.size() != 1) return fail(DUOLM_EINVAL, "debug batch must fit one launch");
  const Plan& P = plans[0];
  const auto& D = R->dims;
  size_t row_bytes = 0;
  const int buf_stage = layer == D.n_layers ? DUOLM_STAGE_LAYER_OUT : stage;
  switch (buf_stage) {
    case DUOLM_STAGE_ATTN_NORM: case DUOLM_STAGE_MLP_NORM: row_bytes = (size_t)D.d_model * 2; break;
    case DUOLM_STAGE_QKV: case DUOLM_STAGE_QK_ROPE: row_bytes = (size_t)R->nqkv * 2; break;
    case DUOLM_STAGE_ATTN: row_bytes = (size_t)D.n_heads * D.head_dim * 2; break;
    case DUOLM_STAGE_SWIGLU: row_bytes = (size_t)D.d_ffn * 2; break;
    default: row_bytes = (size_t)D.d_model * 4;
  }
  if (nbytes != row_bytes * P.T) return fail(DUOLM_EINVAL, "nbytes %llu != %zu", (unsigned long long)nbytes, row_bytes * P.T);
  HIP_TRY(hipSetDevice(R->device));
  Lane& L0 = R->lanes[0];
  if ((rc = ensure_rows(R, L0, P.T))) return rc;
  if ((rc = ensure_meta(R, L0, (int)P.seqs.size(), (int)P.pitems.size(), (int)P.bitems.size(), (int)P.head_rows.size(),
                        (int)P.pages.size())))
    return rc;
  if ((rc = ensure_buf(R, R->d_ids, R->cap_ids, total_ids))) return rc;
  if ((rc = ensure_buf(R, R->d_out, R->cap_out, total_scores))) return rc;
  if ((rc = ensure_buf(R, R->d_inline, R->cap_inline, (int64_t)R->dims.d_model))) return rc;
  R->call_n_inline = 0;
  hipStream_t s = R->stream;
  HIP_TRY(hipMemcpyAsync(R->d_ids, ids.data(), ids.size() * 4, hipMemcpyHostToDevice, s));
  *R->h_err = 0;
  HIP_TRY(hipMemcpyAsync(R->d_err, R->h_err, 4, hipMemcpyHostToDevice, s));
  if ((rc = upload_plan(R, L0, P, s))) return rc;
  Caps c{P.T, (int)P.seqs.size(), (int)P.pitems.size(), (int)P.bitems.size(), (int)P.head_rows.size(), 0, 0, P.TB, 1};
  Enq q{R, &L0, s, nullptr, nullptr};
  q.stop_layer = layer == D.n_layers ? D.n_layers - 1 : layer;
  q.stop_stage = buf_stage;
  enqueue_forward(q, c);
  HIP_TRY(hipGetLastError());
  const void* src = nullptr;
  switch (buf_stage) {
    case DUOLM_STAGE_ATTN_NORM: case DUOLM_STAGE_MLP_NORM: src = L0.Xn; break;
    case DUOLM_STAGE_QKV: case DUOLM_STAGE_QK_ROPE: src = L0.QKV; break;
    case DUOLM_STAGE_ATTN: src = L0.Ob; break;
    case DUOLM_STAGE_SWIGLU: src = L0.Hb; break;
    default: src = L0.X;
  }
  // rows come back in request order -- each sequence's prefix rows, then its
  // branch rows -- not in the packed order (branch region first)
  std::vector<char> packed((size_t)nbytes);
  HIP_TRY(hipMemcpyAsync(packed.data(), src, nbytes, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  char* o = (char*)host_out;
  for (const SeqDesc& sd : P.seqs) {
    const int rows = sd.L + sd.K * sd.M;
    for (int rho = 0; rho < rows; ++rho) {
      const int prow = (rho < sd.L ? sd.row_off : sd.boff) + rho;
      memcpy(o, packed.data() + (size_t)prow * row_bytes, row_bytes);
      o += row_bytes;
    }
  }
  return DUOLM_OK;
}

int duolm_debug_gemm(int32_t epi, const uint16_t* A, const uint16_t* W, void* C, int32_t M, int32_t N, int32_t K,
                     void* stream) {
  if (!A || !W || !C) return fail(DUOLM_EINVAL, "NULL argument");
  if (epi < 0 || epi > 2 || M < 1) return fail(DUOLM_EINVAL, "bad epilogue or M");
  hipStream_t s = (hipStream_t)stream;
  int32_t* dM = nullptr;
  HIP_TRY(hipMalloc((void**)&dM, 4));
  hipError_t e = hipMemcpyAsync(dM, &M, 4, hipMemcpyHostToDevice, s);
  const int ldc = epi == EPI_SWIGLU ? N / 2 : N;
  bool ok = e == hipSuccess && launch_gemm(s, epi, M, A, K, W, K, C, ldc, dM, N, K);
  if (e == hipSuccess) e = hipGetLastError();
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(dM);
  if (e != hipSuccess) return fail(DUOLM_EHIP, "gemm: %s", hipGetErrorString(e));
  if (!ok) return fail(DUOLM_EINVAL, "unsupported GEMM shape N=%d K=%d", N, K);
  return DUOLM_OK;
}

int duolm_copy_device(void* dst, const void* src, uint64_t nbytes, void* stream) {
  if (!dst || !src || nbytes % 16) return fail(DUOLM_EINVAL, "bad copy arguments");
  launch_copy((hipStream_t)stream, dst, src, nbytes);
  HIP_TRY(hipGetLastError());
  return DUOLM_OK;
}

}  // extern "C"
