// Internal descriptors shared by the host planner (ns_api.hip) and the
// kernels (norm_kernels.hip, gemm_kernels.hip). Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsmi {

// Every internal matrix side is padded with zeros to a multiple of PAD so
// that the GEMM kernels never need bounds checks in their main loops. Zero
// padding is exact for this method: the padded rows/columns of X, R, Z, T
// and Q stay zero (diagonal terms are applied only inside the real size).
constexpr int PAD = 256;

// Output element types (match ns_dtype values of the public header).
enum OutType : int { OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2 };

// Row-pair layout of the internal fp16 matrices (rows even, leading
// dimension ld a multiple of 32): element (i, j) sits at
//   (i / 2) * 2 ld + (j / 32) * 64 + (i % 2) * 32 + j % 32,
// i.e. every 128-byte line holds 32 consecutive columns of two neighbouring
// rows. A GEMM K slice of 32 columns over 16 rows is then 8 whole lines
// rather than 16 half lines of a row-major matrix, which lifts the
// global -> LDS copy rate of gfx950 by about 1.5x. User buffers stay
// row-major; the layout of every GEMM operand and output is a flag.
__host__ __device__ inline int64_t pair_index(int64_t i, int64_t j, int64_t ld) {
  return (i >> 1) * 2 * ld + (j >> 5) * 64 + (i & 1) * 32 + (j & 31);
}

// GEMM problem "NT": acc = A * B^T with A (M x K) and B (N x K) row-major
// fp16, leading dimension K for both. Epilogue, evaluated in fp32:
//   v = alpha * acc + beta * C[i][j] + (i == j && i < diag_n ? gamma : 0)
//   D[i][j]  = v                       (dtype out_type, leading dim ldd)
//   D2[i][j] = v + (i == j && i < diag_n ? delta : 0)      (fp16, ld N)
//   DT[j][i] = v                       (fp16, transposed, leading dim M)
// C[i][j] is read with leading dimension ldc and element type c_type
// (fp16 for every internal buffer; a caller's C of any type takes the
// general epilogue). Stores to D are clipped to i < valid_m, j < valid_n.
// Layouts: a_pairs / b_pairs / c_pairs select the row-pair layout (leading
// dimension K for A and B, N for C) instead of row-major; d_pairs does the
// same for D (ld ldd), D2 (ld N) and DT (ld M).
// K-major operands: a_kmajor stores A transposed, as a (K x M) matrix in the
// row-pair layout with leading dimension M (element A[i][k] at
// pair_index(k, i, M)); b_kmajor likewise B as (K x N) with leading
// dimension N. This is how the iteration multiplies by X without keeping
// X^T: Q X takes B = X (K-major), and (Q X)^T = X^T Q takes A = X. At most
// one operand is K-major, never in the symmetric mode, and never B with
// c_is_bt.
// If c_is_bt: the caller guarantees C[i][j] == B[j][i] (C is B^T, which
// needs M <= K), alpha != 0, and the kernel takes beta * C from the B
// slices already in LDS during the K loop instead of reading C again.
// If symmetric: M == N, only tiles on or below the diagonal are computed
// and every stored element (i, j), i >= j, is also stored at (j, i) in D
// and D2, so both come out exactly symmetric.
// The fields a tile needs before its first operand copies come first and
// together (the kernel reads them in one batch of scalar loads); those only
// the epilogue needs follow.
struct GemmDesc {
  const _Float16* A;
  const _Float16* B;
  int tile_begin;      // first logical tile of this problem in the launch
  int tiles_n;         // full: N / BN ; symmetric: M / BM
  int M, N, K;
  int symmetric;
  int c_is_bt;
  int a_pairs, b_pairs;
  int a_kmajor, b_kmajor;
  float alpha, beta;
  int tiles;           // number of tiles of this problem
  const void* C;       // may alias D (same element read then written)
  void* D;
  _Float16* D2;        // optional
  _Float16* DT;        // optional
  int ldd;
  int ldc;             // leading dimension of C (N for internal buffers)
  int c_type;          // OUT_F16 for internal buffers; any OutType for a caller's C
  int valid_m, valid_n;
  int diag_n;
  int out_type;
  int c_pairs, d_pairs;
  float gamma, delta;
};

// Dealing the tiles of one 256 x 256 launch to the 8 XCDs. Hardware hands
// workgroup w to XCD w % 8, and each XCD starts its workgroups in order.
// The problems of a launch are ordered by K, longest first, and the launch's
// logical tiles are cut into segments of equal K (equal tile cost). Within
// a segment, whole rounds of 256 tiles go out as chunks of 32 neighbouring
// tiles (chunk c of a round to XCD c % 8, so each XCD works on tiles that
// share operand panels, and all XCDs on neighbouring chunks of the same
// matrices); the rest of the segment is dealt as evenly as it can be: one
// contiguous piece per XCD, the pieces one tile longer for the XCDs next in
// turn. So every XCD gets the same share of every cost class (to one tile)
// and the end of a long-K class is not left to a few XCDs.
constexpr int MAX_DEAL_SEGS = 16;
struct TileDeal {
  int count;                    // segments; 0 = one segment of the whole launch
  int tiles[MAX_DEAL_SEGS];     // tiles per segment, in logical order
};

// How one 256 x 256 launch hands out its tiles: tiles [0, pool_begin) are
// dealt to workgroups 0 .. pool_begin - 1 by `deal` (over those tiles
// only); tiles [pool_begin, total) form a pool that the remaining
// workgroups claim in order with one atomic counter (zero at launch), and
// `surplus` extra workgroups (which end at once if the pool is empty) let
// the XCDs that run faster claim more of it. pool_begin == total: no pool.
struct GemmCtl {
  TileDeal deal;
  int pool_begin;
  int surplus;
};

// Logical tile of workgroup wg (0 <= wg < total) under deal `dl`; -1 if the
// segments do not cover wg (a malformed deal: the host check refuses it).
__host__ __device__ inline int deal_tile(int wg, int total, const TileDeal& dl) {
  const int x = wg & 7;
  int j = wg >> 3;               // this XCD's j-th workgroup
  int start = 0, turn = 0;       // first tile of the segment, next XCD owed a longer piece
  const int segs = dl.count > 0 ? dl.count : 1;
  for (int s = 0; s < segs; ++s) {
    const int n = dl.count > 0 ? dl.tiles[s] : total;
    const int rounds = n >> 8, rest = n & 255;
    if (j < rounds * 32) return start + (((j >> 5) << 3) + x) * 32 + (j & 31);
    j -= rounds * 32;
    const int q = rest >> 3, e = rest & 7;
    const int mine = q + (((x - turn) & 7) < e ? 1 : 0);
    if (j < mine) {
      int off = start + rounds * 256 + q * x;
      for (int y = 0; y < x; ++y) off += ((y - turn) & 7) < e ? 1 : 0;
      return off + j;
    }
    j -= mine;
    start += n;
    turn = (turn + e) & 7;
  }
  return -1;
}

// Normalisation of one matrix G (m x n, leading dim ldg, dtype g_type):
// x = fp16(g / (||G||_F + eps)). The padded region [0, pm) x [0, pn) in G's
// orientation is written: P[i][j] (ld ldp) and/or PT[j][i] (ld ldpt), zero
// outside the real m x n block. If pairs, P and PT use the row-pair layout
// (with ld ldp / ldpt), else row-major.
struct NormDesc {
  const void* G;
  int64_t ldg;
  int g_type;          // OUT_F32 / OUT_BF16 / OUT_F16 encoding
  int m, n;
  int pm, pn;
  _Float16* P;
  int64_t ldp;
  _Float16* PT;
  int64_t ldpt;
  int pairs;
  float eps;
  // Momentum update fused into the sum-of-squares pass (Muon step): when
  // grad is set, G is the momentum buffer M and the pass first stores
  // M <- fp(beta * M + grad) (fp32 fma, rounded to M's type), then sums the
  // squares of the stored values; the cast pass reads the updated M.
  const void* grad;
  int64_t ldgrad;
  int grad_type;
  float beta;
  float* norm_out;     // optional copy of the norm (device)
  float* norm_slot;    // where the finalize kernel stores the norm
  float* partials;     // chunk partial sums of squares
  int chunk_begin;     // first chunk of this matrix in the sumsq launch
  int chunks;          // chunks of this matrix
  int chunks_n;        // chunks along n
  int tile_begin;      // first 64x64 tile of this matrix in the cast launch
  int tiles;
  int tiles_n;         // tiles along pn
};

// Sum-of-squares chunk: SQ_ROWS x SQ_COLS elements per workgroup.
constexpr int SQ_ROWS = 32;
constexpr int SQ_COLS = 256;
// Cast tile.
constexpr int CAST_TILE = 64;

// Sum of `count` fp16 buffers of `elems` elements each (same layout),
// accumulated in fp32 in index order and rounded once to fp16. It stands in
// for the all-reduce of per-shard partial Gram matrices when one matrix is
// processed as column shards.
constexpr int MAX_SHARDS = 64;
constexpr int REDUCE_ELEMS = 2048;   // elements per workgroup (256 threads x 8)
struct ReduceDesc {
  const _Float16* parts[MAX_SHARDS];
  _Float16* out;
  int64_t elems;       // multiple of 8
  int count;
  int block_begin;     // first workgroup of this reduction in the launch
  int blocks;
};

// Descriptor tables reach the device as kernel arguments: each launch of
// the fill kernel carries TABLE_CHUNK bytes and stores them at `dst`. No
// host staging buffer outlives the call, so a call can be captured into a
// HIP graph and replayed (the bytes are part of the captured launch).
constexpr int TABLE_CHUNK = 2048;
struct TableChunk {
  unsigned char bytes[TABLE_CHUNK];
};

// Launchers (all enqueue on `stream`; return hipSuccess or the launch error).
hipError_t launch_table_fill(unsigned char* dst, const TableChunk& chunk, int bytes,
                             hipStream_t stream);
hipError_t launch_sumsq(const NormDesc* descs, int count, int total_chunks,
                        hipStream_t stream);
hipError_t launch_norm_finalize(const NormDesc* descs, int count,
                                hipStream_t stream);
hipError_t launch_cast(const NormDesc* descs, int count, int total_tiles,
                       hipStream_t stream);
// pool_claims: the launch's pool counter in device memory, zero at launch
// (each launch needs its own; unused without a pool).
hipError_t launch_gemm(const GemmDesc* descs, int count, int total_tiles, const GemmCtl& ctl,
                       int* pool_claims, hipStream_t stream);
constexpr int CLAIM_BYTES = 64;   // room for one launch's pool counter
// The same products on 64 x 64 tiles (tile counts and tile_begin of the
// descriptors in units of 64 x 64 tiles, symmetric problems as the rows of
// their lower triangle); bitwise the same results as launch_gemm. kmajor:
// some descriptor has a K-major operand (selects the kernel that reads them).
hipError_t launch_gemm_small(const GemmDesc* descs, int count, int total_tiles, bool kmajor,
                             hipStream_t stream);
int gemm_small_tile();
hipError_t launch_reduce(const ReduceDesc* descs, int count, int total_blocks,
                         hipStream_t stream);

// Tile edge of the GEMM kernel (BM == BN), and the multiple that every K
// must be (the kernel's LDS ring consumes K in STAGES slices of BK).
int gemm_tile();
int gemm_k_multiple();

}  // namespace nsmi
