// C ABI of the Newton-Schulz library: argument checks, workspace planning,
// stage scheduling and launches. See include/ns.h for the contract.
//
// The stage sequence follows the "Newton-Schulz 变体" page:
//   precision pipeline (section "精度流水线"): norm, scale, fp16 cast;
//   Gram space (section "Gram 空间 NS", equations Z_k and Q_{k+1}) with the
//   restart rule of section "重启机制"; or direct space (section
//   "直接空间 NS"). Every stage is one grouped launch over all matrices of
//   the call. Descriptor tables for all stages are built on the host and
//   copied once per call into the tail of the caller's workspace.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/ns.h"
#include "ns_internal.h"

#define NS_API extern "C" __attribute__((visibility("default")))

namespace nsmi {
namespace {

constexpr size_t ALIGN = 256;
// GEMM stages with fewer 256 x 256 tiles than this run on 64 x 64 tiles.
constexpr int SMALL_STAGE_TILES = 64;
inline size_t align_up(size_t x, size_t a = ALIGN) { return (x + a - 1) / a * a; }
inline int64_t pad_dim(int64_t x) { return (x + PAD - 1) / PAD * PAD; }
inline int ceil_div(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

bool dtype_ok(ns_dtype t) { return t == NS_DT_F32 || t == NS_DT_BF16 || t == NS_DT_F16; }
int out_code(ns_dtype t) { return t == NS_DT_F32 ? OUT_F32 : (t == NS_DT_BF16 ? OUT_BF16 : OUT_F16); }

// ----------------------------------------------------------------- device

enum DevState : int { DEV_UNKNOWN = 0, DEV_OK = 1, DEV_BAD = 2 };
std::mutex g_dev_mu;
std::map<int, int> g_dev_state;
std::map<int, int> g_dev_cus;

ns_status check_device() {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return NS_ERR_UNSUPPORTED;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return NS_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  int& st = g_dev_state[dev];
  if (st == DEV_UNKNOWN) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return NS_ERR_UNSUPPORTED;
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? DEV_OK : DEV_BAD;
    g_dev_cus[dev] = prop.multiProcessorCount;
  }
  return st == DEV_OK ? NS_OK : NS_ERR_UNSUPPORTED;
}

// ---------------------------------------------------------------- upload
// Descriptor tables reach the workspace in one of two ways:
//   * an asynchronous copy from a pinned host staging ring (one copy per
//     call; a slot is reused only after the copy recorded on it has
//     completed), for ordinary calls;
//   * fill-kernel launches whose arguments carry the bytes (TABLE_CHUNK per
//     launch), when the stream is being captured into a HIP graph (the
//     bytes then live in the captured launches, and every replay rewrites
//     the same table) and for the no-allocation entry point (no pinned
//     memory is ever allocated on that path).

struct Slot {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool pending = false;
};
constexpr int RING = 8;
struct Ring {
  Slot slot[RING];
  int next = 0;
};
std::mutex g_up_mu;
std::map<int, Ring> g_rings;

hipError_t upload_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_up_mu);
  Ring& ring = g_rings[dev];
  Slot& s = ring.slot[ring.next];
  ring.next = (ring.next + 1) % RING;
  if (s.pending) {
    e = hipEventSynchronize(s.ev);
    if (e != hipSuccess) return e;
    s.pending = false;
  }
  if (!s.ev) {
    e = hipEventCreateWithFlags(&s.ev, hipEventDisableTiming);
    if (e != hipSuccess) return e;
  }
  if (s.cap < bytes) {
    if (s.host) (void)hipHostFree(s.host);
    s.host = nullptr;
    s.cap = 0;
    const size_t cap = std::max<size_t>(align_up(bytes, 65536), 65536);
    e = hipHostMalloc(&s.host, cap, hipHostMallocPortable);
    if (e != hipSuccess) return e;
    s.cap = cap;
  }
  std::memcpy(s.host, src, bytes);
  e = hipMemcpyAsync(dst, s.host, bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return e;
  e = hipEventRecord(s.ev, stream);
  if (e != hipSuccess) return e;
  s.pending = true;
  return hipSuccess;
}

hipError_t upload_args(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  const unsigned char* from = static_cast<const unsigned char*>(src);
  unsigned char* to = static_cast<unsigned char*>(dst);
  TableChunk chunk;
  for (size_t off = 0; off < bytes; off += TABLE_CHUNK) {
    const size_t n = std::min<size_t>(TABLE_CHUNK, bytes - off);
    const size_t n16 = (n + 15) / 16 * 16;   // the destination is padded to 256 bytes
    std::memcpy(chunk.bytes, from + off, n);
    std::memset(chunk.bytes + n, 0, n16 - n);
    const hipError_t e = launch_table_fill(to + off, chunk, static_cast<int>(n16), stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The copy path unless the stream is capturing (or its status is unknown)
// or the caller must not allocate.
hipError_t upload(void* dst, const void* src, size_t bytes, hipStream_t stream,
                  bool may_allocate = true) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
    (void)hipGetLastError();
    cs = hipStreamCaptureStatusActive;
  }
  if (may_allocate && cs == hipStreamCaptureStatusNone) return upload_copy(dst, src, bytes, stream);
  return upload_args(dst, src, bytes, stream);
}

// ----------------------------------------------------------------- checks

ns_status check_params(const ns_params* p, ns_backend be) {
  if (!p) return NS_ERR_INVALID_ARG;
  if (p->num_steps < 1 || p->num_steps > NS_MAX_STEPS) return NS_ERR_INVALID_ARG;
  if (!p->coeffs) return NS_ERR_INVALID_ARG;
  for (int i = 0; i < 3 * p->num_steps; ++i)
    if (!std::isfinite(p->coeffs[i])) return NS_ERR_INVALID_ARG;
  if (!std::isfinite(p->eps) || p->eps < 0.f) return NS_ERR_INVALID_ARG;
  if (p->num_restarts < 0) return NS_ERR_INVALID_ARG;
  if (p->num_restarts > 0 && !p->restarts) return NS_ERR_INVALID_ARG;
  if (be == NS_GRAM) {
    for (int i = 0; i < p->num_restarts; ++i)
      if (p->restarts[i] < 0 || p->restarts[i] >= p->num_steps) return NS_ERR_INVALID_ARG;
  }
  return NS_OK;
}

ns_status check_matrix_shape(const ns_matrix& a) {
  if (a.m < 1 || a.n < 1 || a.m > NS_MAX_DIM || a.n > NS_MAX_DIM) return NS_ERR_INVALID_ARG;
  if (a.ldg < a.n || a.ldo < a.n) return NS_ERR_INVALID_ARG;
  if (!dtype_ok(a.g_dtype) || !dtype_ok(a.out_dtype)) return NS_ERR_INVALID_ARG;
  return NS_OK;
}

// Byte range [first, last) a row-major (rows, cols, ld) matrix of `es`-byte
// elements spans from `p`.
struct Span { uintptr_t first, last; };
Span span(const void* p, int64_t rows, int64_t cols, int64_t ld, size_t es) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return {a, a + (static_cast<uintptr_t>(rows - 1) * ld + cols) * es};
}
bool overlap(Span x, Span y) { return x.first < y.last && y.first < x.last; }

ns_status check_matrix(const ns_matrix& a) {
  if (!a.g || !a.out) return NS_ERR_INVALID_ARG;
  const ns_status s = check_matrix_shape(a);
  if (s != NS_OK) return s;
  // the output must not overlap the input (the input is read again after
  // outputs of other matrices of the call have been written)
  const size_t gi = a.g_dtype == NS_DT_F32 ? 4 : 2, oi = a.out_dtype == NS_DT_F32 ? 4 : 2;
  if (overlap(span(a.g, a.m, a.n, a.ldg, gi), span(a.out, a.m, a.n, a.ldo, oi)))
    return NS_ERR_INVALID_ARG;
  return NS_OK;
}

// ----------------------------------------------------------------- planning

struct Stage {
  enum Kind { SUMSQ, FINALIZE, CAST, GEMM, REDUCE } kind;
  size_t off;   // byte offset of its descriptors inside the table
  int count;    // descriptors
  int total;    // workgroups (chunks / tiles)
  bool small = false;   // GEMM on 64 x 64 tiles
  bool kmajor = false;  // GEMM with a K-major operand in some descriptor
  GemmCtl ctl{};        // GEMM on 256 x 256 tiles: how its tiles are handed out
  size_t claims_off = 0;  // GEMM on 256 x 256 tiles: its pool counter in the table
  double work;  // algorithmic flops (GEMM) or HBM bytes (normalisation)
};

// Problems of one grouped GEMM launch plus their algorithmic flops.
// Products of one grouped launch. Every operand of the iteration lives in
// the workspace in the row-pair layout; so does every output except the
// final one, which goes to the caller's row-major buffer.
struct Probs {
  std::vector<GemmDesc> d;
  double flops = 0.0;
  void add(GemmDesc g, double f, bool user_output = false, bool user_c = false) {
    g.a_pairs = g.b_pairs = 1;
    g.c_pairs = user_c ? 0 : 1;
    g.d_pairs = user_output ? 0 : 1;
    d.push_back(g);
    flops += f;
  }
};
// s (s + 1) k for a symmetric product, 2 m n k for a general one.
inline double sym_flops(int64_t s, int64_t k) { return double(s) * double(s + 1) * double(k); }
inline double gen_flops(int64_t m, int64_t n, int64_t k) { return 2.0 * m * n * k; }

// A column shard of the working matrix X (s x l, short side first): columns
// [c0, c0 + lc) of X, i.e. columns of G when G is wide and rows of G when it
// is tall. Every entry point but the sharded one uses a single shard.
struct Shard {
  int64_t c0, lc, Lp;      // first column, columns, padded columns
  // Gram: X_i (Sp x Lp) twice (a restart writes Q X into the other one; the
  // products by X read it K-major). Direct: X_i and X_i^T (Lp x Sp) twice
  // (the step's product reads X^T and folds a X from it). Partial Gram
  // matrix (Sp x Sp) of a sharded run.
  size_t X[2], XT[2], Rp;
};

struct MatBuf {   // per-matrix workspace offsets (bytes from ws base)
  int64_t m, n, s, l, Sp, Lp;
  bool tall;
  size_t X, XT[2], R, Z, T, Q[2], A, B;   // X, XT: shard 0's (direct backend)
  std::vector<Shard> sh;
  int chunks, chunks_n, chunk_begin;
};

struct Plan {
  ns_backend backend = NS_GRAM;
  // Muon step (optional): per matrix the gradient added into the momentum
  // in the norm pass, and the update fused into the final product.
  const ns_muon_matrix* muon = nullptr;
  float beta = 0.f, lr = 0.f;
  std::vector<MatBuf> mats;
  std::vector<int> order;          // matrices, largest first
  size_t partials_off = 0, norms_off = 0, table_off = 0, total = 0;
  int total_chunks = 0;
  std::vector<Stage> stages;
  std::vector<unsigned char> table;
};

size_t sq_bytes(int64_t r, int64_t c) { return static_cast<size_t>(r) * c * 2; }

// Workspace layout: per-matrix fp16 buffers, chunk partials, norms, then
// the descriptor table (its size depends only on count and params). With
// shards > 1 (one matrix only) the X buffers and a partial Gram matrix
// exist per shard; shard i has l / shards columns, one more for
// i < l % shards.
void layout(Plan& pl, const ns_matrix* mats, int count, ns_backend be, int shards = 1) {
  size_t off = 0;
  pl.mats.resize(count);
  int chunk_begin = 0;
  for (int i = 0; i < count; ++i) {
    MatBuf& b = pl.mats[i];
    b.m = mats[i].m;
    b.n = mats[i].n;
    b.tall = b.m > b.n;
    b.s = std::min(b.m, b.n);
    b.l = std::max(b.m, b.n);
    b.Sp = pad_dim(b.s);
    b.Lp = pad_dim(b.l);
    const size_t ss = sq_bytes(b.Sp, b.Sp);
    b.sh.resize(shards);
    int64_t c0 = 0;
    for (int k = 0; k < shards; ++k) {
      Shard& h = b.sh[k];
      h.c0 = c0;
      h.lc = b.l / shards + (k < b.l % shards ? 1 : 0);
      c0 += h.lc;
      h.Lp = pad_dim(h.lc);
      const size_t xl = sq_bytes(b.Sp, h.Lp);
      h.X[0] = off; off += xl;
      h.X[1] = h.XT[0] = h.XT[1] = 0;
      if (be == NS_GRAM) {
        h.X[1] = off; off += xl;
      } else {
        h.XT[0] = off; off += xl;
        h.XT[1] = off; off += xl;
      }
      h.Rp = 0;
      if (shards > 1) { h.Rp = off; off += ss; }
    }
    b.X = b.sh[0].X[0];
    b.XT[0] = b.sh[0].XT[0];
    b.XT[1] = b.sh[0].XT[1];
    if (be == NS_GRAM) {
      b.R = off; off += ss;
      b.Z = off; off += ss;
      b.T = off; off += ss;
      b.Q[0] = off; off += ss;
      b.Q[1] = off; off += ss;
    } else {
      b.A = off; off += ss;
      b.B = off; off += ss;
    }
    b.chunks_n = ceil_div(b.n, SQ_COLS);
    b.chunks = ceil_div(b.m, SQ_ROWS) * b.chunks_n;
    b.chunk_begin = chunk_begin;
    chunk_begin += b.chunks;
  }
  pl.total_chunks = chunk_begin;
  pl.partials_off = align_up(off);
  off = pl.partials_off + static_cast<size_t>(chunk_begin) * sizeof(float);
  pl.norms_off = align_up(off);
  off = pl.norms_off + static_cast<size_t>(count) * sizeof(float);
  pl.table_off = align_up(off);
  pl.order.resize(count);
  for (int i = 0; i < count; ++i) pl.order[i] = i;
  std::stable_sort(pl.order.begin(), pl.order.end(), [&](int a, int b) {
    const MatBuf &x = pl.mats[a], &y = pl.mats[b];
    if (x.Sp != y.Sp) return x.Sp > y.Sp;
    return x.Lp > y.Lp;
  });
}

void set_tiles(GemmDesc& d, int T);

struct Arranged {
  int total = 0;        // tiles of the launch
  bool small = false;   // 64 x 64 tile kernel
  bool kmajor = false;  // some descriptor has a K-major operand
  GemmCtl ctl{};        // 256 x 256 kernel: dealt tiles, pool, surplus workgroups
};

// The pool of a 256 x 256 launch: its last tiles, about POOL_WORK of the
// launch's work (a tile's work is its K), claimed in order by whichever
// workgroups get there first; SURPLUS_FRACTION more workgroups than tiles
// give the faster XCDs claimers to spare. Measured on MI355X, XCDs differ
// by up to ~5% in the time they take for the same tiles; the sizes let a
// fast XCD take that much more of the pool. Launches of fewer than
// POOL_MIN_TILES tiles have no pool.
constexpr double POOL_WORK = 0.15;
constexpr double SURPLUS_FRACTION = 0.05;
constexpr int POOL_MIN_TILES = 512;

// Orders the problems of one grouped launch and numbers their tiles:
// problems by K, longest first (the longest-processing-time rule: long
// tiles start early, short ones fill the tail), then by tile count. A launch
// of fewer than SMALL_STAGE_TILES tiles of 256 x 256 (too few to occupy the
// chip) runs on the 64 x 64 tile kernel (force_edge overrides the rule);
// both kernels give the same bits. On the 256 x 256 kernel the last tiles
// form the claimed pool, and the runs of equal K before it become the
// segments by which deal_tile spreads each K class evenly over the XCDs.
Arranged arrange_gemm(std::vector<GemmDesc>& v, int force_edge) {
  Arranged a;
  std::stable_sort(v.begin(), v.end(), [](const GemmDesc& x, const GemmDesc& y) {
    if (x.K != y.K) return x.K > y.K;
    return x.tiles > y.tiles;
  });
  int big = 0;
  for (auto& d : v) big += d.tiles;
  a.small = force_edge ? force_edge == gemm_small_tile() : big < SMALL_STAGE_TILES;
  double work = 0.0;
  for (auto& d : v) {
    if (a.small) set_tiles(d, gemm_small_tile());
    d.tile_begin = a.total;
    a.total += d.tiles;
    a.kmajor = a.kmajor || d.a_kmajor || d.b_kmajor;
    work += double(d.K) * d.tiles;
  }
  if (a.small) return a;
  // the pool: the shortest suffix of the tile order holding POOL_WORK of the work
  int pool_begin = a.total;
  if (a.total >= POOL_MIN_TILES) {
    double rest = POOL_WORK * work;
    for (auto it = v.rbegin(); it != v.rend() && rest > 0.0; ++it) {
      const int take = std::min(it->tiles, static_cast<int>(std::ceil(rest / it->K)));
      pool_begin -= take;
      rest -= double(take) * it->K;
    }
    a.ctl.surplus = (static_cast<int>(std::ceil(SURPLUS_FRACTION * a.total)) + 7) / 8 * 8;
  }
  a.ctl.pool_begin = pool_begin;
  // deal segments: runs of equal K within the dealt tiles [0, pool_begin)
  int n = 0;
  for (size_t i = 0; i < v.size() && v[i].tile_begin < pool_begin; ++i) {
    // past the segment limit, the rest joins the last segment
    if ((i == 0 || v[i].K != v[i - 1].K) && n < MAX_DEAL_SEGS) a.ctl.deal.tiles[n++] = 0;
    a.ctl.deal.tiles[n - 1] += std::min(v[i].tiles, pool_begin - v[i].tile_begin);
  }
  a.ctl.deal.count = n;
  return a;
}

struct Builder {
  Plan& pl;
  unsigned char* ws;   // device base (may be null while sizing)
  explicit Builder(Plan& p, unsigned char* w) : pl(p), ws(w) {}

  _Float16* h(size_t off) const { return reinterpret_cast<_Float16*>(ws + off); }

  template <class D>
  void push(Stage::Kind kind, std::vector<D>& v, int total, double work) {
    if (v.empty()) return;
    Stage st;
    st.kind = kind;
    st.work = work;
    st.off = align_up(pl.table.size(), 64);
    st.count = static_cast<int>(v.size());
    st.total = total;
    pl.table.resize(st.off + v.size() * sizeof(D));
    std::memcpy(pl.table.data() + st.off, v.data(), v.size() * sizeof(D));
    pl.stages.push_back(st);
  }

  // One grouped GEMM launch (see arrange_gemm).
  void gemm_stage(Probs pr, int force_edge = 0) {
    std::vector<GemmDesc>& v = pr.d;
    const Arranged a = arrange_gemm(v, force_edge);
    push(Stage::GEMM, v, a.total, pr.flops);
    if (!v.empty()) {
      Stage& st = pl.stages.back();
      st.small = a.small;
      st.kmajor = a.kmajor;
      st.ctl = a.ctl;
      if (!a.small) {   // the launch's pool counter, zero in every upload of the table
        st.claims_off = align_up(pl.table.size(), 64);
        pl.table.resize(st.claims_off + CLAIM_BYTES, 0);
      }
    }
  }

  // One launch of shard reductions (HBM-bound: every part read once, the
  // sum written once).
  void reduce_stage(std::vector<ReduceDesc>& v) {
    int begin = 0;
    double bytes = 0.0;
    for (auto& d : v) {
      d.block_begin = begin;
      d.blocks = ceil_div(d.elems, REDUCE_ELEMS);
      begin += d.blocks;
      bytes += double(d.elems) * 2.0 * (d.count + 1);
    }
    push(Stage::REDUCE, v, begin, bytes);
  }
};

// Tile counts of a descriptor for tiles of edge T: the lower triangle of
// the tile grid for a symmetric problem, the whole grid otherwise.
void set_tiles(GemmDesc& d, int T) {
  if (d.symmetric) {
    const int t = d.M / T;
    d.tiles_n = t;
    d.tiles = t * (t + 1) / 2;
  } else {
    d.tiles_n = d.N / T;
    d.tiles = (d.M / T) * (d.N / T);
  }
}

GemmDesc gemm(const _Float16* A, const _Float16* B, const _Float16* C, void* D,
              _Float16* D2, _Float16* DT, int64_t M, int64_t N, int64_t K, int64_t ldd,
              int64_t valid_m, int64_t valid_n, int64_t diag_n, int out_type, bool sym,
              float alpha, float beta, float gamma, float delta) {
  GemmDesc d{};
  const int T = gemm_tile();
  d.A = A; d.B = B; d.C = C; d.D = D; d.D2 = D2; d.DT = DT;
  d.M = static_cast<int>(M); d.N = static_cast<int>(N); d.K = static_cast<int>(K);
  d.ldd = static_cast<int>(ldd);
  d.ldc = static_cast<int>(N);
  d.c_type = OUT_F16;
  d.valid_m = static_cast<int>(valid_m); d.valid_n = static_cast<int>(valid_n);
  d.diag_n = static_cast<int>(diag_n);
  d.out_type = out_type;
  d.symmetric = sym ? 1 : 0;
  set_tiles(d, T);
  d.alpha = alpha; d.beta = beta; d.gamma = gamma; d.delta = delta;
  return d;
}

// Marks a product whose C is the transpose of its right operand B (same
// buffer for a symmetric B, or X next to X^T): beta * C is then taken from
// the B slices in LDS. Needs alpha != 0 (the kernel adds beta / alpha * C to
// the accumulators) and M <= K (C's rows are B's columns).
GemmDesc c_from_b(GemmDesc d) {
  d.c_is_bt = (d.C != nullptr && d.beta != 0.f && d.alpha != 0.f && d.M <= d.K) ? 1 : 0;
  return d;
}

inline size_t elem_bytes(ns_dtype t) { return t == NS_DT_F32 ? 4 : 2; }

// Precision pipeline for every matrix: sum of squares and norm over the
// whole matrix, then the scaled cast into X (short side first; also X^T for
// the direct backend), zero-padded, per shard (a shard reads its own block
// of G and the whole matrix's norm: the scalar all-reduce of a sharded run).
void norm_stages(Builder& B, const ns_matrix* mats, float eps) {
  Plan& pl = B.pl;
  const bool with_xt = pl.backend != NS_GRAM;
  std::vector<NormDesc> v, cast;
  int tile_begin = 0;
  double read_bytes = 0.0, write_bytes = 0.0, momentum_bytes = 0.0;
  for (int i : pl.order) {
    const MatBuf& b = pl.mats[i];
    const double elems = double(b.m) * double(b.n);
    read_bytes += elems * elem_bytes(mats[i].g_dtype);
    write_bytes += elems * 2.0 * (with_xt ? 2.0 : 1.0);
    if (pl.muon)   // the momentum pass also reads the gradient and writes M
      momentum_bytes += elems * (elem_bytes(pl.muon[i].grad_dtype) + elem_bytes(mats[i].g_dtype));
    NormDesc d{};
    d.G = mats[i].g;
    d.ldg = mats[i].ldg;
    d.g_type = out_code(mats[i].g_dtype);
    d.m = static_cast<int>(b.m);
    d.n = static_cast<int>(b.n);
    d.eps = eps;
    d.pairs = 1;
    if (pl.muon) {   // M <- beta M + grad in the norm pass
      const ns_muon_matrix& u = pl.muon[i];
      d.grad = u.grad;
      d.ldgrad = u.ld_grad;
      d.grad_type = out_code(u.grad_dtype);
      d.beta = pl.beta;
    }
    d.norm_out = nullptr;
    d.norm_slot = reinterpret_cast<float*>(B.ws + pl.norms_off) + i;
    d.partials = reinterpret_cast<float*>(B.ws + pl.partials_off);
    d.chunk_begin = b.chunk_begin;
    d.chunks = b.chunks;
    d.chunks_n = b.chunks_n;
    v.push_back(d);
    for (const Shard& h : b.sh) {
      NormDesc c = d;
      const size_t off = static_cast<size_t>(h.c0) * elem_bytes(mats[i].g_dtype) *
                         (b.tall ? static_cast<size_t>(mats[i].ldg) : 1);
      c.G = mats[i].g ? static_cast<const unsigned char*>(mats[i].g) + off : nullptr;
      if (!b.tall) {   // G is already short side first: G -> X, G^T -> X^T
        c.n = static_cast<int>(h.lc);
        c.pm = static_cast<int>(b.Sp); c.pn = static_cast<int>(h.Lp);
        c.P = B.h(h.X[0]); c.ldp = h.Lp;
        c.PT = with_xt ? B.h(h.XT[0]) : nullptr; c.ldpt = b.Sp;
      } else {         // tall: G -> X^T, G^T -> X
        c.m = static_cast<int>(h.lc);
        c.pm = static_cast<int>(h.Lp); c.pn = static_cast<int>(b.Sp);
        c.P = with_xt ? B.h(h.XT[0]) : nullptr; c.ldp = b.Sp;
        c.PT = B.h(h.X[0]); c.ldpt = h.Lp;
      }
      c.tiles_n = ceil_div(c.pn, CAST_TILE);
      c.tiles = ceil_div(c.pm, CAST_TILE) * c.tiles_n;
      c.tile_begin = tile_begin;
      tile_begin += c.tiles;
      cast.push_back(c);
    }
  }
  // sumsq chunks are indexed by the chunk_begin of the matrix order in the
  // layout; re-sort the descriptor copy for the chunk search.
  std::vector<NormDesc> by_chunk = v;
  std::sort(by_chunk.begin(), by_chunk.end(),
            [](const NormDesc& a, const NormDesc& b) { return a.chunk_begin < b.chunk_begin; });
  B.push(Stage::SUMSQ, by_chunk, pl.total_chunks, read_bytes + momentum_bytes);
  B.push(Stage::FINALIZE, v, static_cast<int>(v.size()), 0.0);
  B.push(Stage::CAST, cast, tile_begin, read_bytes + write_bytes);
}

// Marks operand A or B of a product as K-major (see GemmDesc).
GemmDesc kmajor(GemmDesc d, bool a, bool b) {
  d.a_kmajor = a ? 1 : 0;
  d.b_kmajor = b ? 1 : 0;
  return d;
}

void final_output(Builder& B, const ns_matrix& mt, const MatBuf& b, const Shard& h,
                  const _Float16* Qm, const _Float16* XT, const _Float16* Xc,
                  const _Float16* XTc, float beta, Probs& out, bool km = false) {
  // wide: out = Q X = Q (X^T)^T                    (M = Sp, N = Lp)
  // tall: out = (Q X)^T = X^T Q^T = X^T Q (Q sym.)  (M = Lp, N = Sp)
  // (direct backend: Q is the step matrix b A + c A^2 and the epilogue adds
  //  beta times X or X^T). A shard writes its own columns (wide) or rows
  // (tall) of the caller's output. km: the operand passed as XT is X
  // itself, read K-major (right operand when wide, left when tall).
  const int ot = out_code(mt.out_dtype);
  const double f = gen_flops(b.s, h.lc, b.s);
  const Plan& pl = B.pl;
  if (pl.muon) {
    // Muon update fused into the epilogue: W <- W - lr * scale * (Q X),
    // W (the caller's buffer, row-major) is both C and D.
    const ns_muon_matrix& u = pl.muon[&b - pl.mats.data()];
    const float alpha = -pl.lr * u.scale;
    const size_t st = elem_bytes(u.param_dtype) * (b.tall ? static_cast<size_t>(u.ld_param) : 1);
    void* w = u.param ? static_cast<unsigned char*>(u.param) + static_cast<size_t>(h.c0) * st
                      : nullptr;
    GemmDesc g = !b.tall ? gemm(Qm, XT, nullptr, w, nullptr, nullptr, b.Sp, h.Lp, b.Sp,
                                u.ld_param, b.m, h.lc, 0, ot, false, alpha, 1.f, 0.f, 0.f)
                         : gemm(XT, Qm, nullptr, w, nullptr, nullptr, h.Lp, b.Sp, b.Sp,
                                u.ld_param, h.lc, b.n, 0, ot, false, alpha, 1.f, 0.f, 0.f);
    g = kmajor(g, km && b.tall, km && !b.tall);
    g.C = w;
    g.ldc = static_cast<int>(u.ld_param);
    g.c_type = ot;
    out.add(g, f, true, true);
    return;
  }
  const size_t step = elem_bytes(mt.out_dtype) * (b.tall ? static_cast<size_t>(mt.ldo) : 1);
  void* o = mt.out ? static_cast<unsigned char*>(mt.out) + static_cast<size_t>(h.c0) * step
                   : nullptr;
  if (!b.tall) {
    GemmDesc g = gemm(Qm, XT, Xc, o, nullptr, nullptr, b.Sp, h.Lp, b.Sp, mt.ldo, b.m, h.lc,
                      0, ot, false, 1.f, beta, 0.f, 0.f);
    out.add(km ? kmajor(g, false, true) : c_from_b(g), f, true);
  } else {
    out.add(kmajor(gemm(XT, Qm, XTc, o, nullptr, nullptr, h.Lp, b.Sp, b.Sp, mt.ldo, h.lc, b.n,
                        0, ot, false, 1.f, beta, 0.f, 0.f), km, false), f, true);
  }
}

void gram_stages(Builder& B, const ns_matrix* mats, const ns_params& p) {
  Plan& pl = B.pl;
  const int K = p.num_steps;
  std::vector<bool> restart(K, false);
  for (int i = 0; i < p.num_restarts; ++i) restart[p.restarts[i]] = true;

  // R = X X^T. A sharded matrix forms one partial Gram matrix per shard
  // (all shards in the same launch, as on separate devices), then their
  // shard-order sum: R = sum_i X_i X_i^T, the exact TP decomposition.
  // xc: which of the two X buffers holds the current X.
  auto syrk_all = [&](int xc) {
    Probs v;
    std::vector<ReduceDesc> red;
    for (int i : pl.order) {
      const MatBuf& b = pl.mats[i];
      if (b.sh.size() == 1) {
        const _Float16* X = B.h(b.sh[0].X[xc]);
        v.add(gemm(X, X, nullptr, B.h(b.R), nullptr, nullptr, b.Sp, b.Sp, b.Lp,
                   b.Sp, b.Sp, b.Sp, 0, OUT_F16, true, 1.f, 0.f, 0.f, 0.f),
              sym_flops(b.s, b.l));
        continue;
      }
      ReduceDesc r{};
      for (const Shard& h : b.sh) {
        v.add(gemm(B.h(h.X[xc]), B.h(h.X[xc]), nullptr, B.h(h.Rp), nullptr, nullptr, b.Sp,
                   b.Sp, h.Lp, b.Sp, b.Sp, b.Sp, 0, OUT_F16, true, 1.f, 0.f, 0.f, 0.f),
              sym_flops(b.s, h.lc));
        r.parts[r.count++] = B.h(h.Rp);
      }
      r.out = B.h(b.R);
      r.elems = b.Sp * b.Sp;
      red.push_back(r);
    }
    B.gemm_stage(v);
    B.reduce_stage(red);
  };

  norm_stages(B, mats, p.eps);
  int xc = 0;
  syrk_all(xc);
  bool q_identity = true;
  int qc = 0;
  for (int k = 0; k < K; ++k) {
    const float a = p.coeffs[3 * k], bk = p.coeffs[3 * k + 1], ck = p.coeffs[3 * k + 2];
    if (restart[k] && !q_identity) {
      // restart: X <- Q X (X read K-major, the product written to the other
      // X buffer), R <- X X^T, Q <- I
      Probs v;
      for (int i : pl.order) {
        const MatBuf& b = pl.mats[i];
        for (const Shard& h : b.sh)   // each shard applies Q to its own columns
          v.add(kmajor(gemm(B.h(b.Q[qc]), B.h(h.X[xc]), nullptr, B.h(h.X[xc ^ 1]), nullptr,
                            nullptr, b.Sp, h.Lp, b.Sp, h.Lp, b.Sp, h.Lp, 0, OUT_F16, false,
                            1.f, 0.f, 0.f, 0.f), false, true),
                gen_flops(b.s, h.lc, b.s));
      }
      B.gemm_stage(v);
      xc ^= 1;
      syrk_all(xc);
      q_identity = true;
    }
    const bool need_r = (k + 1 < K) && !restart[k + 1];
    // Z = b R + c R^2 (and, right after a start or restart, Q = Z + a I)
    {
      Probs v;
      for (int i : pl.order) {
        const MatBuf& b = pl.mats[i];
        _Float16* q2 = q_identity ? B.h(b.Q[qc ^ 1]) : nullptr;
        v.add(c_from_b(gemm(B.h(b.R), B.h(b.R), B.h(b.R), B.h(b.Z), q2, nullptr, b.Sp, b.Sp,
                            b.Sp, b.Sp, b.Sp, b.Sp, b.s, OUT_F16, true, ck, bk, 0.f, a)),
              sym_flops(b.s, b.s));
      }
      B.gemm_stage(v);
    }
    // Q <- Z Q + a Q  and  T = Z R + a R  (both read Z; one launch)
    {
      Probs v;
      for (int i : pl.order) {
        const MatBuf& b = pl.mats[i];
        if (!q_identity)
          v.add(c_from_b(gemm(B.h(b.Z), B.h(b.Q[qc]), B.h(b.Q[qc]), B.h(b.Q[qc ^ 1]), nullptr,
                              nullptr, b.Sp, b.Sp, b.Sp, b.Sp, b.Sp, b.Sp, 0, OUT_F16, true, 1.f,
                              a, 0.f, 0.f)),
                sym_flops(b.s, b.s));
        if (need_r)
          v.add(c_from_b(gemm(B.h(b.Z), B.h(b.R), B.h(b.R), B.h(b.T), nullptr, nullptr, b.Sp,
                              b.Sp, b.Sp, b.Sp, b.Sp, b.Sp, 0, OUT_F16, true, 1.f, a, 0.f,
                              0.f)),
                sym_flops(b.s, b.s));
      }
      B.gemm_stage(v);
    }
    qc ^= 1;
    q_identity = false;
    // R <- T Z + a T   (R_{k+1} = (a I + Z) R (a I + Z)). In exact arithmetic
    // Z T + a T is the same matrix (and would make C = B^T), but with fp16
    // rounding of T and Z this order lands measurably closer to the fp64
    // iteration on square inputs (fp16 model: ~8.7e-3 vs ~1.1e-2 relative on
    // 256 x 256 Gaussians, You table), so C = T is read in the epilogue.
    if (need_r) {
      Probs v;
      for (int i : pl.order) {
        const MatBuf& b = pl.mats[i];
        v.add(gemm(B.h(b.T), B.h(b.Z), B.h(b.T), B.h(b.R), nullptr, nullptr, b.Sp, b.Sp, b.Sp,
                   b.Sp, b.Sp, b.Sp, 0, OUT_F16, true, 1.f, a, 0.f, 0.f),
              sym_flops(b.s, b.s));
      }
      B.gemm_stage(v);
    }
  }
  Probs v;
  for (int i : pl.order) {
    const MatBuf& b = pl.mats[i];
    for (const Shard& h : b.sh)
      final_output(B, mats[i], b, h, B.h(b.Q[qc]), B.h(h.X[xc]), nullptr, nullptr, 0.f, v,
                   true);
  }
  B.gemm_stage(v);
}

void direct_stages(Builder& B, const ns_matrix* mats, const ns_params& p) {
  Plan& pl = B.pl;
  const int K = p.num_steps;
  norm_stages(B, mats, p.eps);
  int xt = 0;
  for (int k = 0; k < K; ++k) {
    const float a = p.coeffs[3 * k], bk = p.coeffs[3 * k + 1], ck = p.coeffs[3 * k + 2];
    Probs v1, v2, v3;
    for (int i : pl.order) {
      const MatBuf& b = pl.mats[i];
      // A = X X^T
      v1.add(gemm(B.h(b.X), B.h(b.X), nullptr, B.h(b.A), nullptr, nullptr, b.Sp, b.Sp, b.Lp,
                  b.Sp, b.Sp, b.Sp, 0, OUT_F16, true, 1.f, 0.f, 0.f, 0.f),
             sym_flops(b.s, b.l));
      // B = b A + c A^2
      v2.add(c_from_b(gemm(B.h(b.A), B.h(b.A), B.h(b.A), B.h(b.B), nullptr, nullptr, b.Sp,
                           b.Sp, b.Sp, b.Sp, b.Sp, b.Sp, 0, OUT_F16, true, ck, bk, 0.f, 0.f)),
             sym_flops(b.s, b.s));
      // X <- a X + B X  (in place; X^T written to the other buffer)
      if (k + 1 < K) {
        v3.add(c_from_b(gemm(B.h(b.B), B.h(b.XT[xt]), B.h(b.X), B.h(b.X), nullptr,
                             B.h(b.XT[xt ^ 1]), b.Sp, b.Lp, b.Sp, b.Lp, b.Sp, b.Lp, 0, OUT_F16,
                             false, 1.f, a, 0.f, 0.f)),
               gen_flops(b.s, b.l, b.s));
      } else {
        final_output(B, mats[i], b, b.sh[0], B.h(b.B), B.h(b.XT[xt]), B.h(b.X), B.h(b.XT[xt]),
                     a, v3);
      }
    }
    B.gemm_stage(v1);
    B.gemm_stage(v2);
    B.gemm_stage(v3);
    xt ^= 1;
  }
}

ns_status build_plan(Plan& pl, const ns_matrix* mats, int count, ns_backend be,
                     const ns_params& p, unsigned char* ws, int shards = 1,
                     const ns_muon_matrix* muon = nullptr, float beta = 0.f, float lr = 0.f) {
  pl.backend = be;
  pl.muon = muon;
  pl.beta = beta;
  pl.lr = lr;
  layout(pl, mats, count, be, shards);
  Builder B(pl, ws);
  if (be == NS_GRAM) gram_stages(B, mats, p);
  else direct_stages(B, mats, p);
  pl.total = align_up(pl.table_off + pl.table.size());
  return NS_OK;
}

// ------------------------------------------------------------ bounds check
// Before any launch, every byte range the kernels of a plan can touch is
// derived from the plan's descriptors the way the kernels address memory
// (see the kernels' load, store and epilogue paths), and must lie inside
// one workspace buffer of the layout or one caller buffer, with write
// permission where it is written. Adjacent buffers are not merged, so an
// overrun into a neighbouring buffer is caught as well. A failure is a
// planner bug: the call returns NS_ERR_INTERNAL and enqueues nothing.

struct Iv {
  uintptr_t lo, hi;
  bool writable;
};

struct Bounds {
  std::vector<Iv> raw;
  std::vector<Iv> rd, wr;   // disjoint after finish(): readable, writable
  std::string err;

  void allow(const void* p, uintptr_t bytes, bool writable) {
    if (!p || bytes == 0) return;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    raw.push_back({a, a + bytes, writable});
  }
  static void merge(std::vector<Iv>& v) {
    std::sort(v.begin(), v.end(), [](const Iv& x, const Iv& y) { return x.lo < y.lo; });
    std::vector<Iv> out;
    for (const Iv& x : v) {
      if (!out.empty() && x.lo < out.back().hi) out.back().hi = std::max(out.back().hi, x.hi);
      else out.push_back(x);
    }
    v.swap(out);
  }
  void finish() {
    for (const Iv& x : raw) {
      rd.push_back(x);
      if (x.writable) wr.push_back(x);
    }
    merge(rd);
    merge(wr);
  }
  static bool inside(const std::vector<Iv>& v, uintptr_t lo, uintptr_t hi) {
    auto it = std::upper_bound(v.begin(), v.end(), lo,
                               [](uintptr_t x, const Iv& y) { return x < y.lo; });
    if (it == v.begin()) return false;
    --it;
    return lo >= it->lo && hi <= it->hi;
  }
  bool fail(const std::string& what) {
    if (err.empty()) err = what;
    return false;
  }
  // elements [lo, hi) of `es` bytes from base
  bool range(const char* what, const void* base, int64_t lo, int64_t hi, size_t es, bool write) {
    if (!err.empty()) return false;
    if (hi <= lo) return true;
    if (!base) return fail(std::string(what) + ": null pointer");
    const uintptr_t a = reinterpret_cast<uintptr_t>(base) + static_cast<uintptr_t>(lo) * es;
    const uintptr_t b = reinterpret_cast<uintptr_t>(base) + static_cast<uintptr_t>(hi) * es;
    if (!inside(write ? wr : rd, a, b)) {
      char buf[256];
      std::snprintf(buf, sizeof(buf), "%s: %s of bytes [%#llx, %#llx) outside every %s buffer",
                    what, write ? "write" : "read", static_cast<unsigned long long>(a),
                    static_cast<unsigned long long>(b), write ? "writable" : "readable");
      return fail(buf);
    }
    return true;
  }
  // the (rows, cols) block at the origin of a matrix with leading dimension
  // ld, row-major or in the row-pair layout
  bool block(const char* what, const void* base, int64_t rows, int64_t cols, int64_t ld,
             bool pairs, size_t es, bool write) {
    if (rows <= 0 || cols <= 0) return true;
    if (pairs && ld % 32) return fail(std::string(what) + ": row-pair layout needs ld % 32 == 0");
    // the last element addressed, as the kernels compute it (also when a
    // block is wider than its leading dimension)
    const int64_t hi = pairs ? pair_index(rows - 1, cols - 1, ld) + 1 : (rows - 1) * ld + cols;
    if (!range(what, base, 0, hi, es, write)) return false;
    // a block wider than its leading dimension wraps into the next rows:
    // inside the buffer, but someone else's elements
    if (cols > ld) return fail(std::string(what) + ": block wider than its leading dimension");
    return true;
  }
};

size_t out_elem(int type) { return type == OUT_F32 ? 4 : 2; }

// Which epilogue the GEMM kernel takes for a descriptor (mirrors the
// dispatch at the end of gemm_nt_kernel).
enum EpiKind { EK_SYM, EK_FAST, EK_GENERAL };
EpiKind epilogue_kind(const GemmDesc& d) {
  if (d.symmetric) return EK_SYM;
  const void* C = d.c_is_bt ? nullptr : d.C;
  const bool row_store_ok = (d.ldd % 8 == 0) && (reinterpret_cast<uintptr_t>(d.D) % 16 == 0);
  if (d.out_type == OUT_F16 && d.valid_m == d.M && d.valid_n == d.N && row_store_ok && !d.D2 &&
      (!C || d.c_type == OUT_F16))
    return EK_FAST;
  return EK_GENERAL;
}

bool check_gemm(const GemmDesc& d, Bounds& B, int T) {
  if (d.M <= 0 || d.N <= 0 || d.K <= 0 || d.M % gemm_tile() || d.N % gemm_tile() ||
      d.K % gemm_k_multiple())
    return B.fail("gemm: M, N or K is not a multiple of the tile");
  if (d.symmetric && d.M != d.N) return B.fail("gemm: symmetric product that is not square");
  const int tm = d.M / T, tn = d.N / T;
  if (d.symmetric ? (d.tiles_n != tm || d.tiles != tm * (tm + 1) / 2)
                  : (d.tiles_n != tn || d.tiles != tm * tn))
    return B.fail("gemm: tile count does not match M and N");
  if (d.valid_m < 0 || d.valid_m > d.M || d.valid_n < 0 || d.valid_n > d.N ||
      d.diag_n < 0 || d.diag_n > std::min(d.M, d.N))
    return B.fail("gemm: valid block or diagonal outside the product");
  if (d.c_is_bt && (!d.C || d.M > d.K || d.alpha == 0.f))
    return B.fail("gemm: C folded from B needs C, M <= K and alpha != 0");
  if (d.a_kmajor || d.b_kmajor) {
    if (d.a_kmajor && d.b_kmajor) return B.fail("gemm: both operands K-major");
    if (d.symmetric) return B.fail("gemm: K-major operand in a symmetric product");
    if ((d.a_kmajor && !d.a_pairs) || (d.b_kmajor && !d.b_pairs))
      return B.fail("gemm: K-major operand not in the row-pair layout");
    if (d.b_kmajor && d.c_is_bt) return B.fail("gemm: C folded from a K-major B");
  }
  // a K-major operand is the (K x width) matrix read by pairs of k rows
  if (d.a_kmajor) B.block("gemm A (K-major)", d.A, d.K, d.M, d.M, true, 2, false);
  else B.block("gemm A", d.A, d.M, d.K, d.K, d.a_pairs, 2, false);
  if (d.b_kmajor) B.block("gemm B (K-major)", d.B, d.K, d.N, d.N, true, 2, false);
  else B.block("gemm B", d.B, d.N, d.K, d.K, d.b_pairs, 2, false);
  const void* C = d.c_is_bt ? nullptr : d.C;
  switch (epilogue_kind(d)) {
    case EK_SYM:
      if (d.out_type != OUT_F16 || (C && d.c_type != OUT_F16))
        return B.fail("gemm: the symmetric epilogue is fp16 only");
      if (d.DT) return B.fail("gemm: DT is ignored by the symmetric epilogue");
      if (C) B.block("gemm C (symmetric)", C, d.M, d.N, d.ldc, d.c_pairs, 2, false);
      B.block("gemm D (symmetric, mirrored)", d.D, d.M, d.N, d.ldd, d.d_pairs, 2, true);
      if (d.D2) B.block("gemm D2", d.D2, d.M, d.N, d.N, d.d_pairs, 2, true);
      break;
    case EK_FAST:
      if (C) B.block("gemm C (tile)", C, d.M, d.N, d.ldc, d.c_pairs, 2, false);
      B.block("gemm D (tile)", d.D, d.M, d.N, d.ldd, d.d_pairs, 2, true);
      if (d.DT) B.block("gemm DT", d.DT, d.N, d.M, d.M, d.d_pairs, 2, true);
      break;
    case EK_GENERAL:
      if (d.D2 || d.DT) return B.fail("gemm: D2 / DT are ignored by the general epilogue");
      if (C) B.block("gemm C (clipped)", C, d.valid_m, d.valid_n, d.ldc, d.c_pairs,
                     out_elem(d.c_type), false);
      B.block("gemm D (clipped)", d.D, d.valid_m, d.valid_n, d.ldd, d.d_pairs,
              out_elem(d.out_type), true);
      break;
  }
  return B.err.empty();
}

// The tiles of one grouped launch: descriptor tile ranges back to back and,
// on the 256 x 256 kernel, every tile handed out exactly once: deal_tile a
// one-to-one map of the first pool_begin workgroups onto tiles
// [0, pool_begin), the rest of the tiles left to the pool.
bool check_deal(const GemmDesc* d, int count, int total, bool small, const GemmCtl& ctl,
                Bounds& B) {
  int next = 0;
  for (int i = 0; i < count; ++i) {
    if (d[i].tile_begin != next) return B.fail("gemm: tile ranges not contiguous");
    next += d[i].tiles;
  }
  if (next != total) return B.fail("gemm: launch size differs from its tiles");
  if (small) return true;
  const int dealt = ctl.pool_begin;
  if (dealt < 0 || dealt > total || ctl.surplus < 0 || (dealt == total && ctl.surplus != 0))
    return B.fail("gemm: pool outside the launch");
  const TileDeal& deal = ctl.deal;
  if (deal.count < 0 || deal.count > MAX_DEAL_SEGS)
    return B.fail("gemm: tile deal with a bad segment count");
  if (deal.count > 0) {
    int sum = 0;
    for (int k = 0; k < deal.count; ++k) {
      if (deal.tiles[k] < 1) return B.fail("gemm: empty tile deal segment");
      sum += deal.tiles[k];
    }
    if (sum != dealt) return B.fail("gemm: tile deal segments do not cover the dealt tiles");
  }
  std::vector<char> seen(static_cast<size_t>(dealt), 0);
  for (int wg = 0; wg < dealt; ++wg) {
    const int t = deal_tile(wg, dealt, deal);
    if (t < 0 || t >= dealt || seen[t]) return B.fail("gemm: tile deal is not one-to-one");
    seen[t] = 1;
  }
  return true;
}

// Checks every descriptor of the plan; `ws` is the workspace base the plan
// was built for.
bool validate_plan(const Plan& pl, const unsigned char* ws, Bounds& B) {
  const size_t tbytes = (pl.table.size() + 15) / 16 * 16;
  B.range("descriptor table", ws, static_cast<int64_t>(pl.table_off),
          static_cast<int64_t>(pl.table_off + tbytes), 1, true);
  for (const Stage& st : pl.stages) {
    const unsigned char* t = pl.table.data() + st.off;
    switch (st.kind) {
      case Stage::GEMM: {
        const GemmDesc* d = reinterpret_cast<const GemmDesc*>(t);
        for (int i = 0; i < st.count; ++i) {
          if (st.small && !st.kmajor && (d[i].a_kmajor || d[i].b_kmajor))
            return B.fail("gemm: K-major operand in a launch of the row-major-only kernel");
          if (!check_gemm(d[i], B, st.small ? gemm_small_tile() : gemm_tile())) return false;
        }
        if (!check_deal(d, st.count, st.total, st.small, st.ctl, B)) return false;
        if (!st.small) {
          int zero[CLAIM_BYTES / sizeof(int)] = {};
          if (st.claims_off % 64 || st.claims_off < st.off ||
              st.claims_off + CLAIM_BYTES > pl.table.size() ||
              std::memcmp(pl.table.data() + st.claims_off, zero, CLAIM_BYTES) != 0)
            return B.fail("gemm: pool counter outside the launch table or not zero");
        }
        break;
      }
      case Stage::SUMSQ:
      case Stage::FINALIZE:
      case Stage::CAST: {
        const NormDesc* d = reinterpret_cast<const NormDesc*>(t);
        int next = 0;
        for (int i = 0; i < st.count; ++i) {
          const NormDesc& n = d[i];
          const size_t ge = out_elem(n.g_type);
          if (st.kind == Stage::SUMSQ) {
            if (n.chunk_begin != next) return B.fail("sumsq: chunk ranges not contiguous");
            next += n.chunks;
            if (n.chunks_n != ceil_div(n.n, SQ_COLS) || n.chunks != ceil_div(n.m, SQ_ROWS) * n.chunks_n)
              return B.fail("sumsq: chunk count does not cover the matrix");
            B.block("sumsq G", n.G, n.m, n.n, n.ldg, false, ge, n.grad != nullptr);
            if (n.grad) B.block("sumsq gradient", n.grad, n.m, n.n, n.ldgrad, false,
                                out_elem(n.grad_type), false);
            B.range("sumsq partials", n.partials, n.chunk_begin, n.chunk_begin + n.chunks, 4, true);
          } else if (st.kind == Stage::FINALIZE) {
            B.range("finalize partials", n.partials, n.chunk_begin, n.chunk_begin + n.chunks, 4,
                    false);
            B.range("finalize norm", n.norm_slot, 0, 1, 4, true);
            if (n.norm_out) B.range("finalize norm copy", n.norm_out, 0, 1, 4, true);
          } else {
            if (n.tile_begin != next) return B.fail("cast: tile ranges not contiguous");
            next += n.tiles;
            if (n.tiles_n != ceil_div(n.pn, CAST_TILE) ||
                n.tiles != ceil_div(n.pm, CAST_TILE) * n.tiles_n)
              return B.fail("cast: tile count does not cover the padded block");
            if (n.m > n.pm || n.n > n.pn) return B.fail("cast: padded block smaller than G");
            B.block("cast G", n.G, n.m, n.n, n.ldg, false, ge, false);
            B.range("cast norm", n.norm_slot, 0, 1, 4, false);
            if (n.P) B.block("cast X", n.P, n.pm, n.pn, n.ldp, n.pairs, 2, true);
            if (n.PT) B.block("cast X^T", n.PT, n.pn, n.pm, n.ldpt, n.pairs, 2, true);
          }
          if (!B.err.empty()) return false;
        }
        if (st.kind != Stage::FINALIZE && next != st.total)
          return B.fail("normalisation: launch size differs from its work");
        break;
      }
      case Stage::REDUCE: {
        const ReduceDesc* d = reinterpret_cast<const ReduceDesc*>(t);
        int next = 0;
        for (int i = 0; i < st.count; ++i) {
          const ReduceDesc& r = d[i];
          if (r.block_begin != next || r.elems % 8 || r.count < 1 || r.count > MAX_SHARDS)
            return B.fail("reduce: malformed descriptor");
          next += r.blocks;
          for (int k = 0; k < r.count; ++k) B.range("reduce part", r.parts[k], 0, r.elems, 2, false);
          B.range("reduce sum", r.out, 0, r.elems, 2, true);
          if (!B.err.empty()) return false;
        }
        if (next != st.total) return B.fail("reduce: launch size differs from its blocks");
        break;
      }
    }
    if (!B.err.empty()) return false;
  }
  return B.err.empty();
}

// The buffers a call may touch: each workspace buffer of the layout, and the
// caller's matrices (inputs read; outputs written; for the Muon step the
// momentum read and written, the gradient read, the parameter read and
// written).
void allow_buffers(Bounds& B, const Plan& pl, const unsigned char* ws, const ns_matrix* mats,
                   int count) {
  for (int i = 0; i < count; ++i) {
    const MatBuf& b = pl.mats[i];
    const size_t ss = sq_bytes(b.Sp, b.Sp);
    for (const Shard& h : b.sh) {
      const size_t xl = sq_bytes(b.Sp, h.Lp);
      B.allow(ws + h.X[0], xl, true);
      if (pl.backend == NS_GRAM) {
        B.allow(ws + h.X[1], xl, true);
      } else {
        B.allow(ws + h.XT[0], xl, true);
        B.allow(ws + h.XT[1], xl, true);
      }
      if (b.sh.size() > 1) B.allow(ws + h.Rp, ss, true);
    }
    if (pl.backend == NS_GRAM) {
      for (size_t off : {b.R, b.Z, b.T, b.Q[0], b.Q[1]}) B.allow(ws + off, ss, true);
    } else {
      B.allow(ws + b.A, ss, true);
      B.allow(ws + b.B, ss, true);
    }
    const ns_matrix& a = mats[i];
    const bool muon = pl.muon != nullptr;
    const size_t gi = elem_bytes(a.g_dtype), oi = elem_bytes(a.out_dtype);
    B.allow(a.g, ((a.m - 1) * a.ldg + a.n) * gi, muon);
    B.allow(a.out, ((a.m - 1) * a.ldo + a.n) * oi, true);
    if (muon) {
      const ns_muon_matrix& u = pl.muon[i];
      B.allow(u.grad, ((u.m - 1) * u.ld_grad + u.n) * elem_bytes(u.grad_dtype), false);
    }
  }
  B.allow(ws + pl.partials_off, static_cast<size_t>(pl.total_chunks) * sizeof(float), true);
  B.allow(ws + pl.norms_off, static_cast<size_t>(count) * sizeof(float), true);
  B.allow(ws + pl.table_off, (pl.table.size() + 15) / 16 * 16, true);
  B.finish();
}

// Deliberate mistakes planted into a built plan (test hook of ns_plan_check;
// never applied on the launch path). Returns false if the plan has no
// descriptor the mistake applies to.
enum Plant {
  PLANT_NONE = 0,
  PLANT_UNCLIPPED_C = 1,    // a caller's C read over the padded tile
  PLANT_UNCLIPPED_D = 2,    // a caller's output written over the padded tile
  PLANT_K_OVERRUN = 3,      // a GEMM reads one K block past its operands
  PLANT_CAST_ROWS = 4,      // the cast writes 64 rows past its padded block
  PLANT_SUMSQ_ROW = 5,      // the norm pass reads one row past G
  PLANT_REDUCE_TAIL = 6,    // a shard reduction runs one block past its parts
  PLANT_KMAJOR_K = 7,       // a K-major operand read from one K block further on
  PLANT_DEAL_LONG = 8,      // a tile deal segment one tile longer than its tiles
};
bool plant_mistake(Plan& pl, const unsigned char* ws, size_t ws_bytes, int plant) {
  auto in_ws = [&](const void* p) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), w = reinterpret_cast<uintptr_t>(ws);
    return a >= w && a < w + ws_bytes;
  };
  for (Stage& st : pl.stages) {
    unsigned char* t = pl.table.data() + st.off;
    if (st.kind == Stage::GEMM) {
      GemmDesc* d = reinterpret_cast<GemmDesc*>(t);
      for (int i = 0; i < st.count; ++i) {
        GemmDesc& g = d[i];
        if (plant == PLANT_UNCLIPPED_C && g.C && !g.c_is_bt && !in_ws(g.C) &&
            (g.valid_m < g.M || g.valid_n < g.N)) {
          g.valid_m = g.M;
          g.valid_n = g.N;
          return true;
        }
        if (plant == PLANT_UNCLIPPED_D && !in_ws(g.D) && (g.valid_m < g.M || g.valid_n < g.N)) {
          g.valid_m = g.M;
          g.valid_n = g.N;
          return true;
        }
        if (plant == PLANT_K_OVERRUN) {
          g.K += gemm_k_multiple();
          return true;
        }
        if (plant == PLANT_DEAL_LONG && !st.small && st.ctl.deal.count > 0) {
          st.ctl.deal.tiles[0] += 1;
          return true;
        }
        if (plant == PLANT_KMAJOR_K && (g.a_kmajor || g.b_kmajor)) {
          // the K-major operand's rows start one K block later (its other
          // operand unchanged)
          const int64_t rows = gemm_k_multiple();
          if (g.a_kmajor) g.A += rows * g.M;
          else g.B += rows * g.N;
          return true;
        }
      }
    } else if (st.kind == Stage::CAST && plant == PLANT_CAST_ROWS && st.count > 0) {
      NormDesc* d = reinterpret_cast<NormDesc*>(t);
      const int old = d[0].tiles;
      d[0].pm += CAST_TILE;
      d[0].tiles = ceil_div(d[0].pm, CAST_TILE) * d[0].tiles_n;
      for (int i = 1; i < st.count; ++i) d[i].tile_begin += d[0].tiles - old;
      st.total += d[0].tiles - old;
      return true;
    } else if (st.kind == Stage::SUMSQ && plant == PLANT_SUMSQ_ROW && st.count > 0) {
      NormDesc* d = reinterpret_cast<NormDesc*>(t);
      d[0].m += 1;
      return true;
    } else if (st.kind == Stage::REDUCE && plant == PLANT_REDUCE_TAIL && st.count > 0) {
      ReduceDesc* d = reinterpret_cast<ReduceDesc*>(t);
      d[0].elems += REDUCE_ELEMS;
      return true;
    }
  }
  return false;
}

// ---------------------------------------------------------------- timing
struct TimedLaunch {
  bool gemm;
  double work;
  hipEvent_t start, end;
};
std::mutex g_time_mu;
bool g_timing = false;
std::vector<TimedLaunch> g_timed;
std::vector<hipEvent_t> g_event_pool;

hipError_t take_event(hipEvent_t* ev) {
  if (!g_event_pool.empty()) {
    *ev = g_event_pool.back();
    g_event_pool.pop_back();
    return hipSuccess;
  }
  return hipEventCreate(ev);
}

bool timing_on() {
  std::lock_guard<std::mutex> lock(g_time_mu);
  return g_timing;
}

// Brackets one launch with events when timing is enabled.
template <class F>
hipError_t timed(bool on, bool gemm_kind, double work, hipStream_t stream, F launch) {
  if (!on) return launch();
  hipEvent_t a = nullptr, b = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_time_mu);
    hipError_t e = take_event(&a);
    if (e == hipSuccess) e = take_event(&b);
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipEventRecord(a, stream);
  if (e == hipSuccess) e = launch();
  if (e == hipSuccess) e = hipEventRecord(b, stream);
  std::lock_guard<std::mutex> lock(g_time_mu);
  g_timed.push_back({gemm_kind, work, a, b});
  return e;
}

// may_allocate == false: no pinned staging memory and no timing events.
ns_status run_plan(const Plan& pl, unsigned char* ws, hipStream_t stream,
                   bool may_allocate = true) {
  unsigned char* table = ws + pl.table_off;
  if (upload(table, pl.table.data(), pl.table.size(), stream, may_allocate) != hipSuccess)
    return NS_ERR_HIP;
  const bool on = may_allocate && timing_on();
  for (const Stage& st : pl.stages) {
    hipError_t e = hipSuccess;
    switch (st.kind) {
      case Stage::SUMSQ:
        e = timed(on, false, st.work, stream, [&] {
          return launch_sumsq(reinterpret_cast<const NormDesc*>(table + st.off), st.count,
                              st.total, stream);
        });
        break;
      case Stage::FINALIZE:
        e = timed(on, false, st.work, stream, [&] {
          return launch_norm_finalize(reinterpret_cast<const NormDesc*>(table + st.off),
                                      st.count, stream);
        });
        break;
      case Stage::CAST:
        e = timed(on, false, st.work, stream, [&] {
          return launch_cast(reinterpret_cast<const NormDesc*>(table + st.off), st.count,
                             st.total, stream);
        });
        break;
      case Stage::GEMM:
        e = timed(on, true, st.work, stream, [&] {
          const GemmDesc* d = reinterpret_cast<const GemmDesc*>(table + st.off);
          return st.small ? launch_gemm_small(d, st.count, st.total, st.kmajor, stream)
                          : launch_gemm(d, st.count, st.total, st.ctl,
                                        reinterpret_cast<int*>(table + st.claims_off), stream);
        });
        break;
      case Stage::REDUCE:
        e = timed(on, false, st.work, stream, [&] {
          return launch_reduce(reinterpret_cast<const ReduceDesc*>(table + st.off), st.count,
                               st.total, stream);
        });
        break;
    }
    if (e != hipSuccess) return NS_ERR_HIP;
  }
  return NS_OK;
}

ns_status check_call(const ns_matrix* mats, int count, ns_backend be, const ns_params* p) {
  if (count < 0) return NS_ERR_INVALID_ARG;
  if (be != NS_GRAM && be != NS_DIRECT) return NS_ERR_INVALID_ARG;
  ns_status s = check_params(p, be);
  if (s != NS_OK) return s;
  if (count > 0 && !mats) return NS_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i) {
    s = check_matrix(mats[i]);
    if (s != NS_OK) return s;
  }
  return NS_OK;
}

ns_status check_shards(const ns_matrix& a, int shards) {
  if (shards < 1 || shards > MAX_SHARDS) return NS_ERR_INVALID_ARG;
  if (shards > std::max(a.m, a.n)) return NS_ERR_INVALID_ARG;
  return NS_OK;
}

ns_status run_batched(const ns_matrix* mats, int count, ns_backend be, const ns_params* p,
                      void* ws, size_t ws_bytes, void* stream, int shards = 1,
                      const ns_muon_matrix* muon = nullptr, float beta = 0.f, float lr = 0.f,
                      bool may_allocate = true) {
  ns_status s = check_call(mats, count, be, p);
  if (s != NS_OK) return s;
  if (count == 0) return NS_OK;
  Plan sizing;
  build_plan(sizing, mats, count, be, *p, nullptr, shards, muon, beta, lr);
  if (!ws || ws_bytes < sizing.total) return NS_ERR_WORKSPACE;
  s = check_device();
  if (s != NS_OK) return s;
  if (reinterpret_cast<uintptr_t>(ws) % ALIGN) return NS_ERR_WORKSPACE;
  Plan pl;
  unsigned char* w = static_cast<unsigned char*>(ws);
  build_plan(pl, mats, count, be, *p, w, shards, muon, beta, lr);
  Bounds bounds;
  allow_buffers(bounds, pl, w, mats, count);
  if (!validate_plan(pl, w, bounds)) return NS_ERR_INTERNAL;
  return run_plan(pl, w, static_cast<hipStream_t>(stream), may_allocate);
}

std::string g_info;

}  // namespace
}  // namespace nsmi

using namespace nsmi;

NS_API const char* ns_status_string(ns_status s) {
  switch (s) {
    case NS_OK: return "NS_OK";
    case NS_ERR_INVALID_ARG: return "NS_ERR_INVALID_ARG";
    case NS_ERR_UNSUPPORTED: return "NS_ERR_UNSUPPORTED";
    case NS_ERR_WORKSPACE: return "NS_ERR_WORKSPACE";
    case NS_ERR_HIP: return "NS_ERR_HIP";
    case NS_ERR_INTERNAL: return "NS_ERR_INTERNAL";
  }
  return "NS_ERR_UNKNOWN";
}

NS_API const char* ns_backend_info(void) {
  char buf[256];
  if (check_device() == NS_OK) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    int cus = 0;
    {
      std::lock_guard<std::mutex> lock(g_dev_mu);
      cus = g_dev_cus[dev];
    }
    std::snprintf(buf, sizeof(buf),
                  "Gram NS / direct NS · kernel=hip-mfma-f16 %dx%d tiles (gfx950, device %d, "
                  "%d CUs)",
                  gemm_tile(), gemm_tile(), dev, cus);
  } else {
    std::snprintf(buf, sizeof(buf),
                  "Gram NS / direct NS · kernel=hip-mfma-f16 (no gfx950 device available)");
  }
  std::lock_guard<std::mutex> lock(g_dev_mu);
  g_info = buf;
  return g_info.c_str();
}

NS_API ns_status ns_backend_status(ns_backend_status_t* out) {
  if (!out) return NS_ERR_INVALID_ARG;
  std::memset(out, 0, sizeof(*out));
  out->device_index = -1;
  out->deterministic = 1;
  out->gemm_tile = gemm_tile();
  out->version = NS_VERSION;
  out->kernel = "hip-mfma-f16 grouped NT GEMM (256x256 tiles, ping-pong waves, row-pair layout)";
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return NS_OK;
  }
  int dev = -1;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return NS_OK;
  }
  out->device_index = dev;
  std::snprintf(out->arch, sizeof(out->arch), "%s", prop.gcnArchName);
  out->compute_units = prop.multiProcessorCount;
  out->clock_mhz = prop.clockRate / 1000;
  out->device_found = check_device() == NS_OK ? 1 : 0;
  return NS_OK;
}

NS_API ns_status ns_timing_enable(int enable) {
  std::lock_guard<std::mutex> lock(g_time_mu);
  g_timing = enable != 0;
  return NS_OK;
}

NS_API ns_status ns_timing_read(ns_timing_report* r) {
  if (!r) return NS_ERR_INVALID_ARG;
  std::vector<TimedLaunch> done;
  {
    std::lock_guard<std::mutex> lock(g_time_mu);
    done.swap(g_timed);
  }
  ns_timing_report out{};
  ns_status st = NS_OK;
  for (const TimedLaunch& t : done) {
    float ms = 0.f;
    if (hipEventSynchronize(t.end) != hipSuccess ||
        hipEventElapsedTime(&ms, t.start, t.end) != hipSuccess) {
      st = NS_ERR_HIP;
      ms = 0.f;
    }
    if (t.gemm) {
      out.gemm_ms += ms;
      out.gemm_launches += 1;
      out.gemm_flops += t.work;
    } else {
      out.norm_ms += ms;
      out.norm_launches += 1;
      out.norm_bytes += t.work;
    }
  }
  {
    std::lock_guard<std::mutex> lock(g_time_mu);
    for (const TimedLaunch& t : done) {
      g_event_pool.push_back(t.start);
      g_event_pool.push_back(t.end);
    }
  }
  *r = out;
  return st;
}

NS_API ns_status ns_workspace_size(const ns_matrix* mats, int count, ns_backend backend,
                                   const ns_params* params, size_t* bytes) {
  if (!bytes || count < 1 || !mats) return NS_ERR_INVALID_ARG;
  if (backend != NS_GRAM && backend != NS_DIRECT) return NS_ERR_INVALID_ARG;
  ns_status s = check_params(params, backend);
  if (s != NS_OK) return s;
  for (int i = 0; i < count; ++i) {
    s = check_matrix_shape(mats[i]);
    if (s != NS_OK) return s;
  }
  Plan pl;
  build_plan(pl, mats, count, backend, *params, nullptr);
  *bytes = pl.total;
  return NS_OK;
}

NS_API ns_status ns_gram(const ns_matrix* mat, const ns_params* params, void* ws,
                         size_t ws_bytes, void* stream) {
  if (!mat) return NS_ERR_INVALID_ARG;
  return run_batched(mat, 1, NS_GRAM, params, ws, ws_bytes, stream);
}

NS_API ns_status ns_gram_sharded_workspace_size(const ns_matrix* mat, int shards,
                                                const ns_params* params, size_t* bytes) {
  if (!bytes || !mat) return NS_ERR_INVALID_ARG;
  ns_status s = check_params(params, NS_GRAM);
  if (s == NS_OK) s = check_matrix_shape(*mat);
  if (s == NS_OK) s = check_shards(*mat, shards);
  if (s != NS_OK) return s;
  Plan pl;
  build_plan(pl, mat, 1, NS_GRAM, *params, nullptr, shards);
  *bytes = pl.total;
  return NS_OK;
}

NS_API ns_status ns_gram_sharded(const ns_matrix* mat, int shards, const ns_params* params,
                                 void* ws, size_t ws_bytes, void* stream) {
  if (!mat) return NS_ERR_INVALID_ARG;
  ns_status s = check_shards(*mat, shards);
  if (s != NS_OK) return s;
  return run_batched(mat, 1, NS_GRAM, params, ws, ws_bytes, stream, shards);
}

// Muon step: the momentum buffer is the NS input (g), the parameter the
// output; the gradient and scale ride along in the plan.
namespace nsmi {
namespace {
ns_status muon_matrices(const ns_muon_matrix* mats, int count, float beta, float lr,
                        std::vector<ns_matrix>& out, bool need_pointers) {
  if (count < 0 || (count > 0 && !mats)) return NS_ERR_INVALID_ARG;
  if (!std::isfinite(beta) || !std::isfinite(lr)) return NS_ERR_INVALID_ARG;
  out.resize(count);
  for (int i = 0; i < count; ++i) {
    const ns_muon_matrix& u = mats[i];
    if (!dtype_ok(u.grad_dtype) || u.ld_grad < u.n || u.ld_momentum < u.n ||
        !std::isfinite(u.scale))
      return NS_ERR_INVALID_ARG;
    if (need_pointers && (!u.grad || !u.momentum || !u.param)) return NS_ERR_INVALID_ARG;
    ns_matrix& a = out[i];
    a.g = u.momentum;
    a.g_dtype = u.momentum_dtype;
    a.m = u.m;
    a.n = u.n;
    a.ldg = u.ld_momentum;
    a.out = u.param;
    a.out_dtype = u.param_dtype;
    a.ldo = u.ld_param;
    ns_status s = need_pointers ? check_matrix(a) : check_matrix_shape(a);
    if (s != NS_OK) return s;
  }
  return NS_OK;
}
}  // namespace
}  // namespace nsmi

NS_API ns_status ns_muon_workspace_size(const ns_muon_matrix* mats, int count,
                                        const ns_params* params, size_t* bytes) {
  if (!bytes || count < 1) return NS_ERR_INVALID_ARG;
  std::vector<ns_matrix> m;
  ns_status s = muon_matrices(mats, count, 0.f, 0.f, m, false);
  if (s == NS_OK) s = check_params(params, NS_GRAM);
  if (s != NS_OK) return s;
  Plan pl;
  build_plan(pl, m.data(), count, NS_GRAM, *params, nullptr, 1, mats, 0.f, 0.f);
  *bytes = pl.total;
  return NS_OK;
}

NS_API ns_status ns_muon_step(const ns_muon_matrix* mats, int count, const ns_params* params,
                              float beta, float lr, void* ws, size_t ws_bytes, void* stream) {
  std::vector<ns_matrix> m;
  ns_status s = muon_matrices(mats, count, beta, lr, m, true);
  if (s != NS_OK) return s;
  return run_batched(m.data(), count, NS_GRAM, params, ws, ws_bytes, stream, 1, mats, beta, lr);
}

NS_API ns_status ns_direct(const ns_matrix* mat, const ns_params* params, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!mat) return NS_ERR_INVALID_ARG;
  return run_batched(mat, 1, NS_DIRECT, params, ws, ws_bytes, stream);
}

NS_API ns_status ns_batched(const ns_matrix* mats, int count, ns_backend backend,
                            const ns_params* params, void* ws, size_t ws_bytes, void* stream) {
  return run_batched(mats, count, backend, params, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------- normalize

namespace nsmi {
namespace {
struct NormPlan {
  size_t partials_off, slot_off, desc_off, total;
  int chunks, chunks_n;
};
NormPlan norm_plan(int64_t m, int64_t n) {
  NormPlan p;
  p.chunks_n = ceil_div(n, SQ_COLS);
  p.chunks = ceil_div(m, SQ_ROWS) * p.chunks_n;
  p.partials_off = 0;
  p.slot_off = align_up(static_cast<size_t>(p.chunks) * sizeof(float));
  p.desc_off = align_up(p.slot_off + sizeof(float));
  p.total = align_up(p.desc_off + sizeof(NormDesc));
  return p;
}
}  // namespace
}  // namespace nsmi

NS_API ns_status ns_normalize_workspace_size(int64_t m, int64_t n, size_t* bytes) {
  if (!bytes || m < 1 || n < 1 || m > NS_MAX_DIM || n > NS_MAX_DIM) return NS_ERR_INVALID_ARG;
  *bytes = norm_plan(m, n).total;
  return NS_OK;
}

NS_API ns_status ns_normalize(const void* g, ns_dtype g_dtype, int64_t m, int64_t n, int64_t ldg,
                              void* x, int64_t ldx, int transpose_tall, float eps,
                              float* norm_out, void* ws, size_t ws_bytes, void* stream) {
  if (!g || !x) return NS_ERR_INVALID_ARG;
  if (m < 1 || n < 1 || m > NS_MAX_DIM || n > NS_MAX_DIM || ldg < n) return NS_ERR_INVALID_ARG;
  if (!dtype_ok(g_dtype)) return NS_ERR_INVALID_ARG;
  if (!std::isfinite(eps) || eps < 0.f) return NS_ERR_INVALID_ARG;
  const bool tr = transpose_tall && m > n;
  if (ldx < (tr ? m : n)) return NS_ERR_INVALID_ARG;
  const NormPlan np = norm_plan(m, n);
  if (!ws || ws_bytes < np.total) return NS_ERR_WORKSPACE;
  ns_status s = check_device();
  if (s != NS_OK) return s;
  unsigned char* w = static_cast<unsigned char*>(ws);
  NormDesc d{};
  d.G = g;
  d.ldg = ldg;
  d.g_type = out_code(g_dtype);
  d.m = static_cast<int>(m);
  d.n = static_cast<int>(n);
  d.pm = static_cast<int>(m);
  d.pn = static_cast<int>(n);
  if (tr) {
    d.PT = static_cast<_Float16*>(x);
    d.ldpt = ldx;
  } else {
    d.P = static_cast<_Float16*>(x);
    d.ldp = ldx;
  }
  d.eps = eps;
  d.norm_out = norm_out;
  d.norm_slot = reinterpret_cast<float*>(w + np.slot_off);
  d.partials = reinterpret_cast<float*>(w + np.partials_off);
  d.chunk_begin = 0;
  d.chunks = np.chunks;
  d.chunks_n = np.chunks_n;
  d.tiles_n = ceil_div(n, CAST_TILE);
  d.tiles = ceil_div(m, CAST_TILE) * d.tiles_n;
  d.tile_begin = 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  NormDesc* dd = reinterpret_cast<NormDesc*>(w + np.desc_off);
  if (upload(dd, &d, sizeof(d), st) != hipSuccess) return NS_ERR_HIP;
  const bool on = timing_on();
  const double in_bytes = double(m) * double(n) * (g_dtype == NS_DT_F32 ? 4.0 : 2.0);
  const double out_bytes = double(m) * double(n) * 2.0;
  if (timed(on, false, in_bytes, st, [&] { return launch_sumsq(dd, 1, np.chunks, st); }) !=
      hipSuccess)
    return NS_ERR_HIP;
  if (timed(on, false, 0.0, st, [&] { return launch_norm_finalize(dd, 1, st); }) != hipSuccess)
    return NS_ERR_HIP;
  if (timed(on, false, in_bytes + out_bytes, st,
            [&] { return launch_cast(dd, 1, d.tiles, st); }) != hipSuccess)
    return NS_ERR_HIP;
  return NS_OK;
}

// ---------------------------------------------------------- building blocks

NS_API ns_status ns_gemm_nt(const void* a, const void* b, const void* c, void* d, int64_t M,
                            int64_t N, int64_t K, float alpha, float beta, float gamma,
                            int symmetric, void* ws, size_t ws_bytes, void* stream) {
  if (!a || !b || !d) return NS_ERR_INVALID_ARG;
  if (M < PAD || N < PAD || K < 1 || M % PAD || N % PAD || K % gemm_k_multiple())
    return NS_ERR_INVALID_ARG;
  if (M > NS_MAX_DIM || N > NS_MAX_DIM || K > NS_MAX_DIM) return NS_ERR_INVALID_ARG;
  if (symmetric && M != N) return NS_ERR_INVALID_ARG;
  if (!c && beta != 0.f) return NS_ERR_INVALID_ARG;
  if (!std::isfinite(alpha) || !std::isfinite(beta) || !std::isfinite(gamma))
    return NS_ERR_INVALID_ARG;
  if (!ws || ws_bytes < NS_UNIT_WORKSPACE_BYTES) return NS_ERR_WORKSPACE;
  ns_status s = check_device();
  if (s != NS_OK) return s;
  GemmDesc g = gemm(static_cast<const _Float16*>(a), static_cast<const _Float16*>(b),
                    static_cast<const _Float16*>(c), d, nullptr, nullptr, M, N, K, N, M, N,
                    std::min(M, N), OUT_F16, symmetric != 0, alpha, c ? beta : 0.f, gamma, 0.f);
  g.tile_begin = 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (upload(ws, &g, sizeof(g), st) != hipSuccess) return NS_ERR_HIP;
  GemmCtl ctl{};   // every tile dealt (one segment), no pool
  ctl.pool_begin = g.tiles;
  if (launch_gemm(static_cast<const GemmDesc*>(ws), 1, g.tiles, ctl, nullptr, st) != hipSuccess)
    return NS_ERR_HIP;
  return NS_OK;
}

// Grouped kernel-level products with every descriptor option (see
// ns_gemm_problem in ns.h). Checks mirror what the kernel's epilogue paths
// honour, so an option the kernel would silently ignore is refused.
namespace nsmi {
namespace {
bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

ns_status grouped_desc(const ns_gemm_problem& q, GemmDesc& g) {
  const int T = gemm_tile();
  if (!q.a || !q.b || !q.d) return NS_ERR_INVALID_ARG;
  if (q.M < T || q.N < T || q.K < gemm_k_multiple() || q.M % T || q.N % T ||
      q.K % gemm_k_multiple() || q.M > NS_MAX_DIM || q.N > NS_MAX_DIM || q.K > NS_MAX_DIM)
    return NS_ERR_INVALID_ARG;
  if (!dtype_ok(q.d_dtype) || (q.c && !dtype_ok(q.c_dtype))) return NS_ERR_INVALID_ARG;
  if (q.valid_m < 0 || q.valid_m > q.M || q.valid_n < 0 || q.valid_n > q.N || q.diag_n < 0 ||
      q.diag_n > std::min(q.M, q.N))
    return NS_ERR_INVALID_ARG;
  // rows of d (and of an unfolded c) hold at least the stored block's width
  if (q.ldd < q.valid_n || (q.c && !q.c_is_bt && q.ldc < q.valid_n)) return NS_ERR_INVALID_ARG;
  if (!std::isfinite(q.alpha) || !std::isfinite(q.beta) || !std::isfinite(q.gamma) ||
      !std::isfinite(q.delta))
    return NS_ERR_INVALID_ARG;
  if (!aligned16(q.a) || !aligned16(q.b)) return NS_ERR_INVALID_ARG;
  if ((q.c_pairs && q.c && q.ldc % 32) || (q.d_pairs && q.ldd % 32)) return NS_ERR_INVALID_ARG;
  const bool fold = q.c_is_bt != 0;
  if (fold && (!q.c || q.M > q.K || q.alpha == 0.f)) return NS_ERR_INVALID_ARG;
  if ((q.a_kmajor && q.b_kmajor) || ((q.a_kmajor || q.b_kmajor) && q.symmetric) ||
      (q.a_kmajor && !q.a_pairs) || (q.b_kmajor && !q.b_pairs) || (q.b_kmajor && fold))
    return NS_ERR_INVALID_ARG;
  const bool full16 = q.d_dtype == NS_DT_F16 && q.valid_m == q.M && q.valid_n == q.N &&
                      q.ldd % 8 == 0 && aligned16(q.d);
  if (q.symmetric) {
    if (q.M != q.N || !full16 || q.dt) return NS_ERR_INVALID_ARG;
    if (q.c && !fold && (q.c_dtype != NS_DT_F16 || q.ldc % 8 || !aligned16(q.c)))
      return NS_ERR_INVALID_ARG;
    if (q.d2 && !aligned16(q.d2)) return NS_ERR_INVALID_ARG;
  } else {
    if (q.d2) return NS_ERR_INVALID_ARG;   // second output only in symmetric mode
    if (q.dt && (!full16 || !aligned16(q.dt) || (q.c && !fold && q.c_dtype != NS_DT_F16)))
      return NS_ERR_INVALID_ARG;
  }
  g = gemm(static_cast<const _Float16*>(q.a), static_cast<const _Float16*>(q.b),
           static_cast<const _Float16*>(q.c), q.d, static_cast<_Float16*>(q.d2),
           static_cast<_Float16*>(q.dt), q.M, q.N, q.K, q.ldd, q.valid_m, q.valid_n, q.diag_n,
           out_code(q.d_dtype), q.symmetric != 0, q.alpha, q.c ? q.beta : 0.f, q.gamma,
           q.delta);
  g.C = q.c;
  g.ldc = static_cast<int>(q.c ? q.ldc : q.N);
  g.c_type = out_code(q.c ? q.c_dtype : NS_DT_F16);
  g.c_is_bt = fold ? 1 : 0;
  g.a_pairs = q.a_pairs ? 1 : 0;
  g.b_pairs = q.b_pairs ? 1 : 0;
  g.c_pairs = q.c_pairs ? 1 : 0;
  g.d_pairs = q.d_pairs ? 1 : 0;
  g.a_kmajor = q.a_kmajor ? 1 : 0;
  g.b_kmajor = q.b_kmajor ? 1 : 0;
  return NS_OK;
}
}  // namespace
}  // namespace nsmi

NS_API ns_status ns_gemm_grouped_workspace_size(int count, size_t* bytes) {
  if (!bytes || count < 1) return NS_ERR_INVALID_ARG;
  // the descriptors, then the launch's pool counter
  *bytes = align_up(align_up(static_cast<size_t>(count) * sizeof(GemmDesc), 64) + CLAIM_BYTES);
  return NS_OK;
}

NS_API ns_status ns_gemm_grouped(const ns_gemm_problem* probs, int count, int tile_edge,
                                 void* ws, size_t ws_bytes, void* stream) {
  if (count < 0 || (count > 0 && !probs)) return NS_ERR_INVALID_ARG;
  if (tile_edge != 0 && tile_edge != gemm_tile() && tile_edge != gemm_small_tile())
    return NS_ERR_INVALID_ARG;
  if (count == 0) return NS_OK;
  Probs v;
  for (int i = 0; i < count; ++i) {
    GemmDesc g{};
    const ns_status s = grouped_desc(probs[i], g);
    if (s != NS_OK) return s;
    v.d.push_back(g);
  }
  size_t need = 0;
  ns_gemm_grouped_workspace_size(count, &need);
  if (!ws || ws_bytes < need || reinterpret_cast<uintptr_t>(ws) % ALIGN) return NS_ERR_WORKSPACE;
  const ns_status s = check_device();
  if (s != NS_OK) return s;
  // the stage planner's order and tile deal (arrange_gemm)
  const Arranged a = arrange_gemm(v.d, tile_edge);
  Bounds B;
  if (!check_deal(v.d.data(), static_cast<int>(v.d.size()), a.total, a.small, a.ctl, B))
    return NS_ERR_INTERNAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the descriptors, then the launch's pool counter (zero)
  const size_t claims_off = align_up(v.d.size() * sizeof(GemmDesc), 64);
  std::vector<unsigned char> bytes(claims_off + CLAIM_BYTES, 0);
  std::memcpy(bytes.data(), v.d.data(), v.d.size() * sizeof(GemmDesc));
  if (upload(ws, bytes.data(), bytes.size(), st) != hipSuccess) return NS_ERR_HIP;
  unsigned char* w = static_cast<unsigned char*>(ws);
  const GemmDesc* dd = reinterpret_cast<const GemmDesc*>(w);
  const int n = static_cast<int>(v.d.size());
  if ((a.small ? launch_gemm_small(dd, n, a.total, a.kmajor, st)
               : launch_gemm(dd, n, a.total, a.ctl, reinterpret_cast<int*>(w + claims_off),
                             st)) != hipSuccess)
    return NS_ERR_HIP;
  return NS_OK;
}

NS_API ns_status ns_syrk(const void* x, int64_t s, int64_t l, void* r, void* ws,
                         size_t ws_bytes, void* stream) {
  if (!x || !r) return NS_ERR_INVALID_ARG;
  return ns_gemm_nt(x, x, nullptr, r, s, s, l, 1.f, 0.f, 0.f, 1, ws, ws_bytes, stream);
}

// --------------------------------------------------------------- self-check

NS_API ns_status ns_plan_check(ns_check_entry entry, const void* mats, int count,
                               ns_backend backend, int shards, const ns_params* params,
                               void* ws, size_t ws_bytes, int plant, char* msg,
                               size_t msg_len) {
  if (msg && msg_len) msg[0] = 0;
  std::vector<ns_matrix> muon_mats;
  const ns_matrix* m = nullptr;
  const ns_muon_matrix* muon = nullptr;
  ns_status s = NS_OK;
  if (entry == NS_CHECK_MUON) {
    muon = static_cast<const ns_muon_matrix*>(mats);
    s = muon_matrices(muon, count, 0.9f, 0.02f, muon_mats, true);
    m = muon_mats.data();
    backend = NS_GRAM;
    shards = 1;
  } else if (entry == NS_CHECK_SHARDED) {
    m = static_cast<const ns_matrix*>(mats);
    if (count != 1 || !m) return NS_ERR_INVALID_ARG;
    s = check_shards(*m, shards);
    backend = NS_GRAM;
  } else if (entry == NS_CHECK_BATCHED) {
    m = static_cast<const ns_matrix*>(mats);
    shards = 1;
  } else {
    return NS_ERR_INVALID_ARG;
  }
  if (s == NS_OK) s = check_call(m, count, backend, params);
  if (s != NS_OK) return s;
  if (count == 0) return NS_OK;
  if (!ws || reinterpret_cast<uintptr_t>(ws) % ALIGN) return NS_ERR_WORKSPACE;
  Plan pl;
  unsigned char* w = static_cast<unsigned char*>(ws);
  build_plan(pl, m, count, backend, *params, w, shards, muon, 0.9f, 0.02f);
  if (ws_bytes == 0) ws_bytes = pl.total;
  if (ws_bytes < pl.total) return NS_ERR_WORKSPACE;
  if (plant != PLANT_NONE && !plant_mistake(pl, w, ws_bytes, plant)) return NS_ERR_UNSUPPORTED;
  Bounds bounds;
  allow_buffers(bounds, pl, w, m, count);
  if (validate_plan(pl, w, bounds)) return NS_OK;
  if (msg && msg_len) std::snprintf(msg, msg_len, "%s", bounds.err.c_str());
  return NS_ERR_INTERNAL;
}

// ------------------------------------------------------ no-allocation entry
// ns_batched for callers that cannot allocate device memory: the workspace
// is this file-scope device array. The host-side name `scratch` is only a
// stand-in for the symbol; each device's copy lives at its own address,
// resolved once per device with hipGetSymbolAddress (with that device
// current), and only that address is ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[NS_NOALLOC_SCRATCH_BYTES];

namespace nsmi {
namespace {
std::mutex g_scratch_mu;
std::map<int, unsigned char*> g_scratch;   // device -> address of its `scratch`

ns_status scratch_address(unsigned char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return NS_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch.find(dev);
  if (it == g_scratch.end()) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return NS_ERR_HIP;
    }
    it = g_scratch.emplace(dev, static_cast<unsigned char*>(p)).first;
  }
  *out = it->second;
  return NS_OK;
}
}  // namespace
}  // namespace nsmi

NS_API ns_status ns_batched_noalloc(const ns_matrix* mats, int count, ns_backend backend,
                                    const ns_params* params, void* stream) {
  ns_status s = check_call(mats, count, backend, params);
  if (s != NS_OK) return s;
  if (count == 0) return NS_OK;
  Plan sizing;
  build_plan(sizing, mats, count, backend, *params, nullptr);
  if (sizing.total > NS_NOALLOC_SCRATCH_BYTES) return NS_ERR_WORKSPACE;
  s = check_device();
  if (s != NS_OK) return s;
  unsigned char* ws = nullptr;
  s = scratch_address(&ws);
  if (s != NS_OK) return s;
  return run_batched(mats, count, backend, params, ws, NS_NOALLOC_SCRATCH_BYTES, stream, 1,
                     nullptr, 0.f, 0.f, /*may_allocate=*/false);
}
