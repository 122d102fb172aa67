// Host-side AddressSanitizer check of libduolm's host code.  The library's
// host code (api.cpp: validation, the request packer, the launch planner,
// descriptor upload, graph cache, execution lanes, sessions) is compiled with
// the sanitizer for host code only; device code is unchanged.  Every buffer
// handed to the library is allocated at exactly its stated size, so a read or
// write past it lands in the sanitizer's redzone.
//
//   host_asan pack            packer only, no GPU: random structured requests,
//                             checked against a plain assembly here, every
//                             thread count, and the error paths
//   host_asan score WEIGHTS   executor on GPU 0: random batches scored through
//                             every entry point and mode, sessions, errors
//
// Prints "ok ..." and exits 0 when every check passed; any mismatch exits 1,
// and a sanitizer report aborts the process.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <vector>

#include "duolm.h"

namespace {

int g_fail = 0;

#define CHECK(cond, ...)                                              \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "check failed (%s:%d): ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);                              \
      std::fprintf(stderr, " [%s]\n", duolm_last_error());            \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

struct Rng {  // xorshift64*
  uint64_t s;
  explicit Rng(uint64_t seed) : s(seed * 0x9E3779B97F4A7C15ull + 1) {}
  uint64_t next() {
    s ^= s >> 12;
    s ^= s << 25;
    s ^= s >> 27;
    return s * 0x2545F4914F6CDD1Dull;
  }
  int uni(int lo, int hi) { return lo + (int)(next() % (uint64_t)(hi - lo + 1)); }  // [lo, hi]
};

// A heap array of exactly n elements (n = 0 gives a 1-element allocation
// that must not be read).
template <class T>
struct Exact {
  std::unique_ptr<T[]> p;
  size_t n;
  explicit Exact(size_t n_) : p(new T[n_ ? n_ : 1]), n(n_) {}
  T* get() { return p.get(); }
};

// ---------------------------------------------------------------------------
// packer
// ---------------------------------------------------------------------------
struct HistReq {
  std::vector<int32_t> vids, feedback, foff, cands;
  int n_items = 0, item_len = 0, n_cand = 1, cand_len = 0;
};

struct Batch {
  std::vector<int32_t> instr, header;
  int32_t marker = 7;
  std::vector<HistReq> reqs;
  std::vector<duolm_history> hist;
  duolm_template tpl{};
  void finish() {
    hist.clear();
    for (auto& r : reqs) {
      duolm_history h{};
      h.n_items = r.n_items;
      h.item_len = r.item_len;
      h.item_vids = r.vids.data();
      h.feedback = r.feedback.data();
      h.feedback_off = r.foff.data();
      h.cand_vids = r.cands.data();
      h.n_cand = r.n_cand;
      h.cand_len = r.cand_len;
      hist.push_back(h);
    }
    tpl.instruction = instr.data();
    tpl.n_instruction = (int32_t)instr.size();
    tpl.marker = marker;
    tpl.cand_header = header.data();
    tpl.n_cand_header = (int32_t)header.size();
  }
};

Batch random_batch(Rng& g, int max_req) {
  Batch b;
  for (int i = g.uni(0, 5); i > 0; --i) b.instr.push_back(g.uni(0, 999));
  for (int i = g.uni(0, 3); i > 0; --i) b.header.push_back(g.uni(0, 999));
  b.marker = g.uni(0, 999);
  for (int q = g.uni(1, max_req); q > 0; --q) {
    HistReq r;
    r.n_items = g.uni(0, 8);
    r.item_len = g.uni(0, 3);
    const int iv = r.item_len ? r.item_len : 1;
    for (int i = 0; i < r.n_items * iv; ++i) r.vids.push_back(1000 + g.uni(0, 499));
    r.foff.push_back(0);
    for (int i = 0; i < r.n_items; ++i) {
      for (int f = g.uni(0, 4); f > 0; --f) r.feedback.push_back(g.uni(0, 999));
      r.foff.push_back((int32_t)r.feedback.size());
    }
    r.n_cand = g.uni(1, 20);
    r.cand_len = g.uni(0, 3);
    const int cv = r.cand_len ? r.cand_len : 1;
    for (int i = 0; i < r.n_cand * cv; ++i) r.cands.push_back(1000 + g.uni(0, 499));
    b.reqs.push_back(std::move(r));
  }
  b.finish();
  return b;
}

// The input layout written out plainly: instruction, then per history item
// the marker, its vids and its feedback, then the header, then the candidates.
void assemble(const Batch& b, std::vector<int32_t>& ids, std::vector<int32_t>& L, std::vector<int32_t>& K,
              std::vector<int32_t>& M) {
  for (const auto& r : b.reqs) {
    const size_t start = ids.size();
    ids.insert(ids.end(), b.instr.begin(), b.instr.end());
    const int iv = r.item_len ? r.item_len : 1;
    for (int i = 0; i < r.n_items; ++i) {
      ids.push_back(b.marker);
      ids.insert(ids.end(), r.vids.begin() + i * iv, r.vids.begin() + (i + 1) * iv);
      ids.insert(ids.end(), r.feedback.begin() + r.foff[i], r.feedback.begin() + r.foff[i + 1]);
    }
    ids.insert(ids.end(), b.header.begin(), b.header.end());
    L.push_back((int32_t)(ids.size() - start));
    K.push_back(r.n_cand);
    M.push_back(r.cand_len ? r.cand_len : 1);
    ids.insert(ids.end(), r.cands.begin(), r.cands.end());
  }
}

int run_pack() {
  Rng g(1);
  int batches = 0;
  for (int it = 0; it < 300; ++it) {
    Batch b = random_batch(g, it % 10 == 0 ? 400 : 40);
    const int n = (int)b.reqs.size();
    std::vector<int32_t> want, wL, wK, wM;
    assemble(b, want, wL, wK, wM);
    int64_t n_ids = -1;
    bool empty_prefix = false;
    for (int32_t l : wL) empty_prefix |= l == 0;
    if (empty_prefix) {  // no instruction, history or header: refused, nothing written
      Exact<int32_t> ids(want.size()), L(n), K(n), M(n);
      CHECK(duolm_packed_size(&b.tpl, b.hist.data(), n, &n_ids) == DUOLM_EINVAL, "empty prefix accepted");
      CHECK(duolm_pack_requests(&b.tpl, b.hist.data(), n, 4, ids.get(), (int64_t)want.size(), L.get(), K.get(),
                                M.get()) == DUOLM_EINVAL,
            "empty prefix packed");
      ++batches;
      continue;
    }
    CHECK(duolm_packed_size(&b.tpl, b.hist.data(), n, &n_ids) == DUOLM_OK, "packed_size");
    CHECK(n_ids == (int64_t)want.size(), "packed_size %lld != %zu", (long long)n_ids, want.size());
    for (int nt : {0, 1, 3, 8, 64}) {
      Exact<int32_t> ids(want.size()), L(n), K(n), M(n);
      const int rc = duolm_pack_requests(&b.tpl, b.hist.data(), n, nt, ids.get(), (int64_t)want.size(), L.get(),
                                         K.get(), M.get());
      CHECK(rc == DUOLM_OK, "pack_requests rc %d (threads %d)", rc, nt);
      if (rc != DUOLM_OK) continue;
      CHECK(std::memcmp(ids.get(), want.data(), want.size() * 4) == 0, "ids differ (threads %d)", nt);
      CHECK(std::memcmp(L.get(), wL.data(), n * 4) == 0 && std::memcmp(K.get(), wK.data(), n * 4) == 0 &&
                std::memcmp(M.get(), wM.data(), n * 4) == 0,
            "lengths differ (threads %d)", nt);
    }
    // one id short of the output: refused before anything is written
    if (!want.empty()) {
      Exact<int32_t> ids(want.size() - 1), L(n), K(n), M(n);
      CHECK(duolm_pack_requests(&b.tpl, b.hist.data(), n, 4, ids.get(), (int64_t)want.size() - 1, L.get(), K.get(),
                                M.get()) == DUOLM_EINVAL,
            "short output accepted");
    }
    ++batches;
  }
  // malformed requests and templates
  Batch b = random_batch(g, 5);
  int64_t n_ids;
  const int n = (int)b.reqs.size();
  CHECK(duolm_packed_size(nullptr, b.hist.data(), n, &n_ids) == DUOLM_EINVAL, "NULL template");
  CHECK(duolm_packed_size(&b.tpl, b.hist.data(), 0, &n_ids) == DUOLM_EINVAL, "no requests");
  CHECK(duolm_packed_size(&b.tpl, nullptr, n, &n_ids) == DUOLM_EINVAL, "NULL requests");
  duolm_history h = b.hist[0];
  h.n_items = -1;
  CHECK(duolm_packed_size(&b.tpl, &h, 1, &n_ids) == DUOLM_EINVAL, "negative items");
  h = b.hist[0];
  h.n_cand = 0;
  CHECK(duolm_packed_size(&b.tpl, &h, 1, &n_ids) == DUOLM_EINVAL, "no candidates");
  h = b.hist[0];
  h.cand_len = DUOLM_MAX_CAND_LEN + 1;
  CHECK(duolm_packed_size(&b.tpl, &h, 1, &n_ids) == DUOLM_EINVAL, "cand_len over the limit");
  {
    HistReq r;
    r.n_items = 2;
    r.vids = {1000, 1001};
    r.feedback = {1, 2, 3};
    r.foff = {0, 3, 2};  // decreasing
    r.cands = {1002};
    Batch bad;
    bad.reqs.push_back(r);
    bad.finish();
    CHECK(duolm_packed_size(&bad.tpl, bad.hist.data(), 1, &n_ids) == DUOLM_EINVAL, "decreasing feedback offsets");
  }
  std::printf("ok pack: %d random batches, 5 thread counts each, error paths\n", batches);
  return g_fail ? 1 : 0;
}

// ---------------------------------------------------------------------------
// executor (GPU)
// ---------------------------------------------------------------------------
struct Req {
  std::vector<int32_t> prefix, cands;
  int m = 1;
};

std::vector<duolm_request> as_requests(const std::vector<Req>& rs) {
  std::vector<duolm_request> out;
  for (const auto& r : rs) {
    duolm_request q{};
    q.ids = r.prefix.data();
    q.prefix_len = (int32_t)r.prefix.size();
    q.cand_ids = r.cands.data();
    q.n_cand = (int32_t)(r.cands.size() / r.m);
    q.cand_len = r.m;
    out.push_back(q);
  }
  return out;
}

size_t n_scores(const std::vector<Req>& rs) {
  size_t n = 0;
  for (const auto& r : rs) n += r.cands.size() / r.m;
  return n;
}

int score(duolm_ranker* R, const std::vector<Req>& rs, std::vector<float>& out, int mode, int graph, int lanes) {
  auto q = as_requests(rs);
  Exact<float> s(n_scores(rs));
  duolm_opts o{};
  o.mode = mode;
  o.use_graph = graph;
  o.max_lanes = lanes;
  const int rc = duolm_score_batch(R, q.data(), (int32_t)q.size(), s.get(), &o);
  if (rc == DUOLM_OK) out.assign(s.get(), s.get() + s.n);
  return rc;
}

int run_score(const char* path) {
  duolm_ranker* R = nullptr;
  CHECK(duolm_load_ranker(path, 0, &R) == DUOLM_OK, "load %s", path);
  if (!R) return 1;
  duolm_dims D{};
  CHECK(duolm_get_dims(R, &D) == DUOLM_OK, "dims");
  const int V = D.vocab, NV = 500;
  Rng g(2);
  {
    std::vector<uint16_t> table((size_t)NV * D.d_model);
    for (auto& x : table) x = (uint16_t)(0x2000 + g.uni(0, 0x0fff)) | (uint16_t)(g.uni(0, 1) << 15);  // |x| < 0.06
    CHECK(duolm_load_vid_table(R, table.data(), NV) == DUOLM_OK, "vid table");
  }
  auto rand_req = [&](int max_l, int max_k, int max_m) {
    Req r;
    r.prefix.resize(g.uni(1, max_l));
    for (auto& x : r.prefix) x = g.uni(0, 4) ? g.uni(0, V - 1) : V + g.uni(0, NV - 1);
    r.m = g.uni(1, max_m);
    r.cands.resize((size_t)g.uni(1, max_k) * r.m);
    for (auto& x : r.cands) x = V + g.uni(0, NV - 1);
    return r;
  };
  int calls = 0;
  for (int it = 0; it < 24; ++it) {
    // batches of 1 to 12 requests; every fourth is large enough (>= 2048 rows)
    // to run as two lanes
    std::vector<Req> rs;
    const bool big = it % 4 == 3;
    for (int q = g.uni(1, big ? 12 : 6); q > 0; --q) rs.push_back(big ? rand_req(300, 40, 1) : rand_req(200, 30, 3));
    if (big)
      while (true) {
        size_t rows = 0;
        for (auto& r : rs) rows += r.prefix.size() + r.cands.size();
        if (rows >= 2048 && rs.size() >= 2) break;
        rs.push_back(rand_req(300, 40, 1));
      }
    std::vector<float> a, b, c, d;
    CHECK(score(R, rs, a, DUOLM_MODE_MIS, 1, 0) == DUOLM_OK, "graph");
    CHECK(score(R, rs, b, DUOLM_MODE_MIS, 0, 0) == DUOLM_OK, "eager");
    CHECK(score(R, rs, c, DUOLM_MODE_MIS, 1, 1) == DUOLM_OK, "one lane");
    CHECK(a == b && a == c, "graph, eager and one-lane scores differ (batch %d)", it);
    if (it % 3 == 0) {
      CHECK(score(R, rs, d, DUOLM_MODE_INDEPENDENT, 1, 0) == DUOLM_OK, "independent");
      CHECK(a == d, "MIS and independent scores differ (batch %d)", it);
    }
    // the same requests packed in host memory
    {
      const int n = (int)rs.size();
      Exact<int32_t> L(n), K(n), M(n);
      size_t tot = 0;
      for (auto& r : rs) tot += r.prefix.size() + r.cands.size();
      Exact<int32_t> ids(tot);
      size_t o = 0;
      for (int i = 0; i < n; ++i) {
        L.get()[i] = (int32_t)rs[i].prefix.size();
        K.get()[i] = (int32_t)(rs[i].cands.size() / rs[i].m);
        M.get()[i] = rs[i].m;
        std::memcpy(ids.get() + o, rs[i].prefix.data(), rs[i].prefix.size() * 4);
        o += rs[i].prefix.size();
        std::memcpy(ids.get() + o, rs[i].cands.data(), rs[i].cands.size() * 4);
        o += rs[i].cands.size();
      }
      Exact<float> s(n_scores(rs));
      CHECK(duolm_score_packed(R, L.get(), K.get(), M.get(), n, ids.get(), s.get(), nullptr) == DUOLM_OK, "packed");
      CHECK(std::vector<float>(s.get(), s.get() + s.n) == a, "packed scores differ (batch %d)", it);
    }
    calls += it % 3 == 0 ? 5 : 4;
  }
  // error paths: nothing written, the handle stays usable
  {
    std::vector<Req> rs = {rand_req(50, 5, 1)};
    std::vector<float> base, out;
    CHECK(score(R, rs, base, DUOLM_MODE_MIS, 1, 0) == DUOLM_OK, "base");
    Req bad = rs[0];
    bad.prefix[0] = V + NV;
    CHECK(score(R, {bad}, out, DUOLM_MODE_MIS, 1, 0) == DUOLM_ERANGE, "out-of-range id");
    bad = rs[0];
    bad.prefix.clear();
    CHECK(score(R, {bad}, out, DUOLM_MODE_MIS, 1, 0) == DUOLM_EINVAL, "empty prefix");
    auto q = as_requests(rs);
    q[0].cand_len = DUOLM_MAX_CAND_LEN + 1;
    Exact<float> s(64);
    CHECK(duolm_score_batch(R, q.data(), 1, s.get(), nullptr) == DUOLM_EINVAL, "cand_len over the limit");
    q = as_requests(rs);
    CHECK(duolm_score_batch(R, q.data(), 1, nullptr, nullptr) == DUOLM_EINVAL, "NULL scores");
    CHECK(score(R, rs, out, DUOLM_MODE_MIS, 1, 0) == DUOLM_OK && out == base, "handle unusable after errors");
  }
  // sessions: appends in random chunks equal one-call scoring of the prefix so far
  {
    CHECK(duolm_kv_pool_init(R, 64 * 64) == DUOLM_OK, "pool");
    std::vector<duolm_session*> ss(3, nullptr);
    for (auto& s : ss) CHECK(duolm_session_create(R, &s) == DUOLM_OK, "session");
    std::vector<Req> full(3);
    for (int step = 0; step < 6; ++step) {
      std::vector<int32_t> n_new(3), n_cand(3), ids;
      std::vector<Req> now;
      for (int i = 0; i < 3; ++i) {
        Req add = rand_req(70, 12, 1);
        n_new[i] = step % 3 == 2 ? 0 : (int32_t)add.prefix.size();
        n_cand[i] = (int32_t)add.cands.size();
        full[i].prefix.insert(full[i].prefix.end(), add.prefix.begin(), add.prefix.begin() + n_new[i]);
        if (full[i].prefix.empty()) {  // candidates need a prefix
          n_new[i] = (int32_t)add.prefix.size();
          full[i].prefix = add.prefix;
        }
        ids.insert(ids.end(), add.prefix.begin(), add.prefix.begin() + n_new[i]);
        ids.insert(ids.end(), add.cands.begin(), add.cands.end());
        Req r;
        r.prefix = full[i].prefix;
        r.cands = add.cands;
        now.push_back(r);
      }
      Exact<int32_t> ex_ids(ids.size());
      std::memcpy(ex_ids.get(), ids.data(), ids.size() * 4);
      Exact<float> s(n_scores(now));
      CHECK(duolm_session_step(R, ss.data(), 3, n_new.data(), n_cand.data(), nullptr, ex_ids.get(), s.get(),
                               nullptr) == DUOLM_OK,
            "session step %d", step);
      std::vector<float> want;
      CHECK(score(R, now, want, DUOLM_MODE_MIS, 1, 0) == DUOLM_OK, "one-call");
      CHECK(std::vector<float>(s.get(), s.get() + s.n) == want, "session step %d differs from one call", step);
    }
    int64_t before = 0, after = 0;
    CHECK(duolm_kv_pool_free_pages(R, &before) == DUOLM_OK, "free pages");
    duolm_session_free(ss[0]);
    CHECK(duolm_kv_pool_free_pages(R, &after) == DUOLM_OK && after > before, "pages returned");
    // the other two sessions are freed with the ranker
  }
  duolm_free_ranker(R);
  std::printf("ok score: %d scoring calls over 24 random batches, packed path, error paths, 6 session steps\n", calls);
  return g_fail ? 1 : 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc >= 2 && !std::strcmp(argv[1], "pack")) return run_pack();
  if (argc >= 3 && !std::strcmp(argv[1], "score")) return run_score(argv[2]);
  std::fprintf(stderr, "usage: %s pack | score WEIGHTS\n", argv[0]);
  return 2;
}
