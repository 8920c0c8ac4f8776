// Grouped fp16 MFMA GEMM "NT" for gfx950: every product of the iteration.
//
// One launch runs the tiles of many independent problems (one per matrix of
// a batch, sometimes two per matrix); each workgroup finds its problem from
// the descriptor table. All products of the method reduce to this one form:
//
//   acc = A * B^T, A (M x K) and B (N x K) row-major fp16, fp32 accumulation
//
// because every Gram-space matrix (R, Z, T, Q) is symmetric in exact
// arithmetic and is stored exactly symmetric (lower-triangle tiles computed,
// then mirrored), so a symmetric right operand B equals B^T; and Q X reads
// X as a K-major right operand (the direct-space step keeps X^T instead).
//
// Uses on the "Newton-Schulz 变体" page: the Gram product R = X X^T
// (section "Gram 空间 NS", SYRK: lower-triangle tiles only, about half the
// tiles), Z = b R + c R^2 (equation Z_k, epilogue alpha = c, beta = b,
// C = R, plus the fused Q = Z + a I output on the first step after a start
// or restart), Q <- Z Q + a Q (equation Q_{k+1}), the R recurrence
// T = Z R + a R, R <- T Z + a T, the restart and output products Q X, and
// the direct-space step X <- a X + (b A + c A^2) X (section "直接空间 NS").
//
// Kernel structure (gfx950):
//   * 256 x 256 workgroup tile, 8 waves in two groups of four (one wave of
//     each group per SIMD); each wave owns a 128 x 64 sub-tile of 32x32x16
//     fp16 MFMAs with fp32 accumulators;
//   * operand tiles move global -> LDS by the buffer-load-to-LDS path (no
//     register staging), through a four-stage ring of 256 x 32 slices;
//     group 0 copies the A slices, group 1 the B slices;
//   * ping-pong schedule: in each phase one group issues its 16 MFMAs back
//     to back while the other group reads the next slice's fragments and
//     issues its copies, with one barrier per phase, so the MFMA pipe of
//     every SIMD is fed by one wave while the other waits on memory;
//   * internal matrices use the row-pair layout (see ns_internal.h): a
//     32-column slice of 16 rows is 8 whole 128-byte lines, which the copy
//     path moves about 1.5x faster than 16 half lines of a row-major matrix;
//   * LDS rows are 64 bytes; the 16-byte chunks are XOR-swizzled by
//     (row / 4) % 4 so the 16 lanes served per cycle by a 128-bit LDS read
//     (16 consecutive rows) hit 16 distinct bank groups;
//   * workgroup ids are remapped so each XCD (8 per MI355X, one L2 each)
//     works on runs of 32 neighbouring tiles that share operand panels, and
//     every XCD gets the same share of the tiles of each K (deal_tile); the
//     last tiles of a launch are claimed from a pool instead, so the XCDs
//     that run faster do more of them;
//   * either operand may instead be K-major (stored K x width in the
//     row-pair layout, see km_off): X serves as the right operand of Q X,
//     or as the left one of X^T Q, without a transposed copy; its slices
//     are copied by pairs of k rows and read with transposing LDS reads;
//   * a diagonal tile of a symmetric product computes only its 36 stored
//     32 x 32 blocks (on or below the diagonal), 5 per wave of group 1 and 4
//     per wave of group 0 (diag_block), so its two MFMA phases per K slice
//     issue 10 and 8 MFMAs instead of 16 and 16;
//   * epilogue arithmetic is written out (explicit fused multiply-adds, the
//     fp32 value held before its conversion), so every code path computing
//     an element rounds it the same way.
// A second kernel runs the same products on 64 x 64 tiles, for stages whose
// few 256 x 256 tiles would leave most of the chip idle; it produces the same
// bits (see gemm_small_kernel).
#include "ns_internal.h"

#include <type_traits>

namespace nsmi {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int THREADS = WAVES_M * WAVES_N * 64;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int KCH = BK / 8;  // 16-byte chunks per tile row
  static constexpr int KSTEPS = BK / 16;
  static constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK;
  static_assert(BM == BN, "square tiles (symmetric mode mirrors tiles)");
  static_assert(KCH == 4, "swizzle assumes 64-byte LDS rows");
};

// Workgroup tile 256 x 256, K slices of 32, eight waves of 128 x 64.
using MainCfg = Cfg<256, 256, 32, 128, 64>;
constexpr int STAGES = 4;      // LDS ring depth (K must be a multiple of 4 * 32)

// Physical 16-byte chunk of logical chunk c in LDS row `row` (64-byte rows).
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor (gfx9 layout): 48-bit base, stride 0, size in bytes;
// reads past `bytes` return zero.
__device__ __forceinline__ i32x4 make_rsrc(const void* p, uint32_t bytes) {
  // every word is wave-uniform; readfirstlane keeps the descriptor in SGPRs,
  // which the copy instruction requires
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  i32x4 r = {__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a))),
             __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xffff)),
             __builtin_amdgcn_readfirstlane(static_cast<int>(bytes)), 0x00020000};
  return r;
}

// One wave-wide global -> LDS copy of 16 bytes per lane: lane i's bytes land
// at LDS byte address lds_addr + 16 i. Written as inline assembly so that
// the only waits on it are the explicit vmcnt waits of the main loop (the
// compiler would otherwise wait for every in-flight copy before any LDS
// read). M0 is not used for anything else in this kernel.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff,
                                           uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr_of(const _Float16* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const _Float16*)(p)));
}

// s_waitcnt immediate (gfx9): vmcnt in bits [3:0] and [15:14]; expcnt and
// lgkmcnt left at their maxima, i.e. only vector-memory completions waited.
constexpr int vmcnt_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Logical tile of a full problem -> (ti, tj): bands of 4 tile rows, walked
// column by column, so 32 consecutive tiles span 4 A panels and 8 B panels.
__device__ __forceinline__ void decode_full(int t, int tiles_m, int tiles_n,
                                            int& ti, int& tj) {
  constexpr int BAND = 4;
  const int band = t / (BAND * tiles_n);
  const int rem = t - band * BAND * tiles_n;
  const int rows = min(BAND, tiles_m - band * BAND);
  ti = band * BAND + rem % rows;
  tj = rem / rows;
}

// Logical tile of a symmetric problem -> (ti, tj), tj <= ti: the lower
// triangle of the T x T tile grid cut into bands of 4 tile rows, each band
// walked column by column (like full problems), so 32 consecutive tiles span
// about 4 A panels and 8 B panels. A full band b starts at 8b^2 + 2b.
__device__ __forceinline__ void decode_lower(int t, int T, int& ti, int& tj) {
  constexpr int BAND = 4;
  int b = 0, start = 0;
  for (;;) {                                   // at most T / 4 iterations
    const int rows = min(BAND, T - BAND * b);
    const int size = (BAND * b + 1) * rows + rows * (rows - 1) / 2;
    if (t < start + size || rows <= 0) break;
    start += size;
    ++b;
  }
  const int rows = min(BAND, T - BAND * b);
  int r = t - start;
  const int first = (BAND * b + 1) * rows;    // columns 0 .. 4b hold `rows` tiles each
  if (r < first) {
    tj = r / rows;
    ti = BAND * b + r % rows;
    return;
  }
  r -= first;
  int u = 1;                                   // column 4b + u holds rows - u tiles
  while (r >= rows - u) {
    r -= rows - u;
    ++u;
  }
  tj = BAND * b + u;
  ti = BAND * b + u + r;
}

__device__ __forceinline__ int find_problem(const GemmDesc* descs, int count, int t) {
  int lo = 0, hi = count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (descs[mid].tile_begin <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  // round to nearest even; NaN kept quiet
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

#define NSMI_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ NSMI_GLOBAL T* gmem(T* p) {
  return (NSMI_GLOBAL T*)(p);
}
template <class T>
__device__ __forceinline__ const NSMI_GLOBAL T* gmem(const T* p) {
  return (const NSMI_GLOBAL T*)(p);
}

// Compile-time loop: f(integral_constant<int, I>) for I in [B, E). Keeps
// accumulator indices constant so the accumulators stay in registers.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

struct Epi {
  float alpha, beta, gamma, delta;
  const void* C;
  int ldc, c_type;
  void* D;
  _Float16* D2;
  _Float16* DT;
  int M, N, ldd, diag_n, valid_m, valid_n, out_type;
  int c_pairs, d_pairs;   // row-pair layout of C / of D, D2, DT
  int row0, col0;   // this lane's first row / column inside the tile
};

// Element (i, j) of a matrix with leading dimension ld, row-major or in the
// row-pair layout.
__device__ __forceinline__ int64_t lidx(int pairs, int64_t i, int64_t j, int64_t ld) {
  return pairs ? pair_index(i, j, ld) : i * ld + j;
}

// Typed element access for the general epilogue (type fixed at compile time).
template <int T>
__device__ __forceinline__ float load_typed(const void* p, int64_t k) {
  if constexpr (T == OUT_F16) return static_cast<float>(gmem(static_cast<const _Float16*>(p))[k]);
  else if constexpr (T == OUT_F32) return gmem(static_cast<const float*>(p))[k];
  else return __uint_as_float(static_cast<uint32_t>(gmem(static_cast<const uint16_t*>(p))[k]) << 16);
}
template <int T>
__device__ __forceinline__ void store_typed(void* p, int64_t k, float v) {
  if constexpr (T == OUT_F16) gmem(static_cast<_Float16*>(p))[k] = static_cast<_Float16>(v);
  else if constexpr (T == OUT_F32) gmem(static_cast<float*>(p))[k] = v;
  else gmem(static_cast<uint16_t*>(p))[k] = to_bf16_bits(v);
}

// The fp32 value of an epilogue is held in a register before it is
// converted to the output type: otherwise the compiler may fuse the last
// multiply-add with the conversion (a mixed-precision fma rounding the exact
// result once to fp16) in some inlined copies and not in others, and rare
// ties would round differently depending on which copy computed an element.
__device__ __forceinline__ float fp32_value(float x) {
  asm("" : "+v"(x));
  return x;
}

// MFMA 32x32 output layout: register r of lane l holds row
// 8*(r/4) + 4*(l/32) + r%4 and column l%32 of each 32x32 block.

// General epilogue for outputs that are not fp16 internal buffers: a
// caller's buffer of any type, clipped to the real (valid_m, valid_n)
// block, with an optional C of any type (read only inside that block; it
// may be the output itself). Types are template parameters, and each
// block's C values are loaded together before any is used, so one memory
// latency is paid per block rather than per element.
//   v = alpha * acc + beta * C + (gamma on the real diagonal)
template <class Cf, int OT, int CT, class Acc>
__device__ __forceinline__ void epilogue_output_t(const Acc& acc, const Epi& e) {
  static_for<0, Cf::FM>([&](auto I) {
    static_for<0, Cf::FN>([&](auto J) {
      const floatx16& a = acc[I][J];
      const int col = e.col0 + J * 32;
      const int rb0 = e.row0 + I * 32;
      const bool col_ok = col < e.valid_n;
      float c[16];
      if constexpr (CT >= 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rb0 + (r / 4) * 8 + (r % 4);
          c[r] = (col_ok && row < e.valid_m)
                     ? load_typed<CT>(e.C, lidx(e.c_pairs, row, col, e.ldc)) : 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rb0 + (r / 4) * 8 + (r % 4);
        float x = e.alpha * a[r];
        if constexpr (CT >= 0) x = __builtin_fmaf(e.beta, c[r], x);
        if (row == col && col < e.diag_n) x += e.gamma;
        if (col_ok && row < e.valid_m)
          store_typed<OT>(e.D, lidx(e.d_pairs, row, col, e.ldd), fp32_value(x));
      }
    });
  });
}

template <class Cf, class Acc>
__device__ __forceinline__ void epilogue_output(const Acc& acc, const Epi& e) {
  const int ct = e.C ? e.c_type : -1;
#define NSMI_EPI_OUT(OT)                                                            \
  if (e.out_type == OT) {                                                          \
    if (ct == OUT_F16) epilogue_output_t<Cf, OT, OUT_F16>(acc, e);                \
    else if (ct == OUT_F32) epilogue_output_t<Cf, OT, OUT_F32>(acc, e);           \
    else if (ct == OUT_BF16) epilogue_output_t<Cf, OT, OUT_BF16>(acc, e);         \
    else epilogue_output_t<Cf, OT, -1>(acc, e);                                    \
    return;                                                                        \
  }
  NSMI_EPI_OUT(OUT_F16)
  NSMI_EPI_OUT(OUT_F32)
  NSMI_EPI_OUT(OUT_BF16)
#undef NSMI_EPI_OUT
}

// ------------------------------------------------------------------ fast epilogue
// After a 32-lane swap each lane holds 8 consecutive rows of one column (16
// bytes): stored directly for transposed outputs, and staged in LDS (the
// operand ring is idle after the main loop) for row-major ones, which read
// it back transposed so that each lane again stores 16 bytes.

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  // one v_cvt_pk_f16_f32: both values rounded to nearest even, as two
  // separate conversions would round them
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}
__device__ __forceinline__ float lo_h(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
__device__ __forceinline__ float hi_h(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}
// After lane_swap(x, y): lanes 32..63 of x hold lanes 0..31 of the old y and
// lanes 0..31 of y hold lanes 32..63 of the old x (v_permlane32_swap).
__device__ __forceinline__ void lane_swap(uint32_t& x, uint32_t& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  x = r[0];
  y = r[1];
}

// Output staging: the tile transposed. Tile column c is the 512-byte LDS
// row c; its 16-byte chunk k holds tile rows 8k..8k+7 and sits at physical
// chunk k ^ stage_sw(c). Both access patterns spread over the 16 bank groups:
// a staging write (32 consecutive columns, two chunks each) and a transposing
// read (16 columns: 4 per 16-lane group, at column offsets 0-3, 8-11, 16-19,
// 24-27 or their +4 shifts).
__device__ __forceinline__ int stage_sw(int c) { return (c & 31) ^ (((c >> 4) & 1) << 2); }
__device__ __forceinline__ uint32_t stage_off(int c, int chunk) {
  return static_cast<uint32_t>(c) * 512u + (static_cast<uint32_t>(chunk ^ stage_sw(c)) << 4);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;

// ds_read_b64_tr_b16: within each 16-lane group, lane j supplies the address
// of four consecutive 16-bit values M[j][0..3]; lane i receives
// M[4q + i/4][i%4] in slot q.
__device__ __forceinline__ u32x2 lds_read_tr(const lds_char* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// K-major operand slices. A K-major operand is stored as (K x width) in the
// row-pair layout, so one pair of k rows over a tile's columns is a single
// contiguous run of whole 128-byte lines (32 columns of both rows each); a
// K slice of 32 is 16 such pairs, one copy instruction per pair (1 KB for
// 256 columns). In LDS, pair q of a slice takes PAIR halves: the 64-half
// unit of column block c (both rows, 32 columns each) sits at unit
// c ^ (q & 1), and the two 16-column halves of each row are swapped when
// bit 2 of q is set. A fragment is then read with two transposing reads,
// each giving a lane four consecutive k of one column; the 32 lanes of a
// half wave touch two pairs at opposite unit parity and the lanes 8 k
// apart touch the other halves of the rows, so the reads spread over all
// bank groups.
template <int PAIR>
__device__ __forceinline__ int km_off(int q, int r, int c, int w) {
  return q * PAIR + ((c ^ (q & 1)) << 6) + (r << 5) + (w ^ (((q >> 2) & 1) << 4));
}

// Offset (halves) from a slice's first pair at the tile's first column of
// the 16 bytes that copy slot s (0..7) of unit u of pair q must fetch so
// that they land where km_off reads them (width = leading dimension).
__device__ __forceinline__ int64_t km_src(int q, int u, int s, int64_t width) {
  const int c = u ^ (q & 1);
  const int w = ((s & 3) * 8) ^ (((q >> 2) & 1) << 4);
  return static_cast<int64_t>(q) * 2 * width + c * 64 + (s >> 2) * 32 + w;
}

// MFMA operand fragment of 32 operand rows (slice columns col .. col + 31)
// at k step ks from a K-major slice: lane l receives k 16 ks + 8 (l / 32)
// + 0..7 of column col + l % 32, as a row-major slice's 16-byte read gives.
// A 16-lane group covers 16 columns and four k per transposing read: its
// lane j points at k row kb + j / 4, columns 4 (j % 4) .. + 3.
template <int PAIR>
__device__ __forceinline__ half8 km_frag(const _Float16* S, int col, int ks, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int n = col + 16 * (g & 1) + 4 * (j & 3);
  const int c = n >> 5, w = n & 31;
  const lds_char* const Sl = (const lds_char*)(S);
  const int k0 = 16 * ks + 8 * (g >> 1) + (j >> 2);
  const int k1 = k0 + 4;
  const u32x2 v0 = lds_read_tr(Sl + 2 * km_off<PAIR>(k0 >> 1, k0 & 1, c, w));
  const u32x2 v1 = lds_read_tr(Sl + 2 * km_off<PAIR>(k1 >> 1, k1 & 1, c, w));
  const u32x4 x = {v0[0], v0[1], v1[0], v1[1]};
  return __builtin_bit_cast(half8, x);
}

// Diagonal tile of a symmetric product: of its 8 x 8 blocks of 32 x 32 only
// the 36 with row block bi >= column block bj are stored (the others are
// their mirror). Wave wn of group 1 takes blocks (wn .. wn + 4, wn); wave wn
// of group 0 takes the rest of column wn, rows wn + 5 .. 7 (3 - wn blocks),
// and column 7 - wn, rows 7 - wn .. 7 (wn + 1 blocks): 5 + 4 blocks per pair
// of waves, so the two MFMA phases of a K slice issue 10 and 8 MFMAs.
__device__ __forceinline__ void diag_block(int grp, int wn, int b, int& bi, int& bj) {
  if (grp == 1) {
    bi = wn + b;
    bj = wn;
    return;
  }
  const int na = 3 - wn;
  if (b < na) {
    bi = wn + 5 + b;
    bj = wn;
  } else {
    bj = 7 - wn;
    bi = bj + (b - na);
  }
}

enum EpiMode { EPI_SYM_OFFDIAG, EPI_SYM_DIAG, EPI_FULL, EPI_FULL_C };

// Fast epilogue for fp16 outputs inside internal (padded, aligned) buffers:
//   * v = alpha acc + beta C + gamma (real diagonal) in fp32, rounded once;
//   * a 32-lane swap gives each lane eight consecutive rows of one column
//     (16 bytes): stored as is for the transposed outputs (symmetric mirror,
//     or DT), and staged in LDS for the row-major output;
//   * row-major stores read the staging with transposing LDS reads, so each
//     lane stores eight consecutive columns of one row (16 bytes);
//   * symmetric C read from its transpose in 16-byte chunks;
//   * diagonal tiles: elements above the diagonal take the value computed
//     at the mirrored position, so the tile comes out exactly symmetric; the
//     second output D2 = D + delta I takes delta on the fp32 diagonal value.
template <class Cf, int MODE, class Acc>
__device__ __forceinline__ void epilogue_tile(const Acc& acc, const Epi& e, _Float16* S,
                                              float* sdiag, int lane, int wm, int wn,
                                              int m0, int n0, _Float16* T, int ldT,
                                              _Float16* T2) {
  static_assert(Cf::BM == 256 && Cf::BN == 256, "tile-wide staging is 256 x 256");
  constexpr bool SYM = MODE == EPI_SYM_OFFDIAG || MODE == EPI_SYM_DIAG;
  lds_char* const Sl = (lds_char*)(S);
  const int h = lane >> 5;
  static_for<0, Cf::FM>([&](auto I) {
    static_for<0, Cf::FN>([&](auto J) {
      int brow = wm * Cf::WM + I * 32, bcol = wn * Cf::WN + J * 32;
      if constexpr (MODE == EPI_SYM_DIAG) {
        // diagonal tile: accumulator slot I + 4 J holds block diag_block(.)
        constexpr int b = I + 4 * J;
        if (b >= (wm == 1 ? 5 : 4)) return;
        int bi, bj;
        diag_block(wm, wn, b, bi, bj);
        brow = bi * 32;
        bcol = bj * 32;
      }
      const floatx16& a = acc[I][J];
      const int lcol = bcol + (lane & 31);                      // tile-local column
      const int lrow0 = brow;                                   // tile-local block row
      const int col = n0 + lcol, rbase = m0 + lrow0;            // global
      uint32_t P[4][2];
      static_for<0, 2>([&](auto GP) {
        constexpr int g0 = 2 * GP;
        float c[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        if constexpr (SYM) {
          if (e.C) {
            const u32x4 cv = *gmem(reinterpret_cast<const u32x4*>(
                static_cast<const _Float16*>(e.C) + lidx(e.c_pairs, col, rbase + 8 * (g0 + h), e.ldc)));
            uint32_t x0 = cv[0], x1 = cv[1], y0 = cv[2], y1 = cv[3];
            lane_swap(x0, y0);
            lane_swap(x1, y1);
            c[0][0] = lo_h(x0); c[0][1] = hi_h(x0); c[0][2] = lo_h(x1); c[0][3] = hi_h(x1);
            c[1][0] = lo_h(y0); c[1][1] = hi_h(y0); c[1][2] = lo_h(y1); c[1][3] = hi_h(y1);
          }
        }
        // The diagonal term exists only in 32 x 32 blocks on the diagonal;
        // the test is uniform, so other blocks skip the per-element compare.
        const bool bdiag = MODE != EPI_SYM_OFFDIAG && rbase == col - (lane & 31);
        static_for<0, 2>([&](auto GG) {
          constexpr int g = g0 + GG;
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = rbase + g * 8 + h * 4 + q;
            // fused multiply-adds written out, so that every code path
            // computing an element rounds it the same way
            float x = e.alpha * a[g * 4 + q];
            if constexpr (SYM) x = __builtin_fmaf(e.beta, c[GG][q], x);
            if constexpr (MODE == EPI_FULL_C)
              x = __builtin_fmaf(e.beta, static_cast<float>(gmem(static_cast<const _Float16*>(
                                     e.C))[lidx(e.c_pairs, row, col, e.ldc)]), x);
            v[q] = x;
          }
          if (bdiag) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int row = rbase + g * 8 + h * 4 + q;
              if (e.gamma != 0.f && row == col && col < e.diag_n) v[q] += e.gamma;
              if constexpr (MODE == EPI_SYM_DIAG)
                if (row == col) sdiag[row - m0] = v[q];
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = fp32_value(v[q]);
          P[g][0] = pack_h2(v[0], v[1]);
          P[g][1] = pack_h2(v[2], v[3]);
        });
        // eight consecutive rows of column `col` per lane: rows
        // rbase + 8 (g0 + h) .. + 7
        uint32_t x0 = P[g0][0], x1 = P[g0][1], y0 = P[g0 + 1][0], y1 = P[g0 + 1][1];
        lane_swap(x0, y0);
        lane_swap(x1, y1);
        const u32x4 out = {x0, x1, y0, y1};
        *(__attribute__((address_space(3))) u32x4*)(Sl + stage_off(lcol, (lrow0 >> 3) + g0 + h)) = out;
        // (the mirror of a symmetric tile is stored from the staging below)
        if constexpr (MODE == EPI_FULL || MODE == EPI_FULL_C) {
          if (T) {   // transposed copy
            const int64_t off = lidx(e.d_pairs, col, rbase + 8 * (g0 + h), ldT);
            *gmem(reinterpret_cast<u32x4*>(T + off)) = out;
            if (T2) *gmem(reinterpret_cast<u32x4*>(T2 + off)) = out;
          }
        }
      });
    });
  });
  // Diagonal tiles mirror across waves: wait for every wave's staging.
  // Otherwise each wave reads back only what it staged itself.
  if constexpr (MODE == EPI_SYM_DIAG) __syncthreads();
  // Row-major copy of this wave's 128 x 64 block, 16 rows x 32 columns per
  // instruction: 16-lane group gq covers columns 8 gq .. 8 gq + 7, lane j of
  // it one row. Source lane j = 4 q + a of a transposing read points at tile
  // rows 4a .. 4a + 3 of column q (+4 for the second read).
  _Float16* D = static_cast<_Float16*>(e.D);
  const int gq = lane >> 4, j = lane & 15, qa = j >> 2, aa = j & 3;
  static_for<0, Cf::WM / 16>([&](auto RB) {
    static_for<0, Cf::WN / 32>([&](auto CB) {
      const int R0 = wm * Cf::WM + RB * 16, C0 = wn * Cf::WN + CB * 32;
      const int chunk = (R0 >> 3) + (aa >> 1);
      const int c1 = C0 + 8 * gq + qa;
      const u32x2 t1 = lds_read_tr(Sl + stage_off(c1, chunk) + (aa & 1) * 8);
      const u32x2 t2 = lds_read_tr(Sl + stage_off(c1 + 4, chunk) + (aa & 1) * 8);
      u32x4 val = {t1[0], t1[1], t2[0], t2[1]};
      const int lr = R0 + j, lc = C0 + 8 * gq;   // this lane's row, first column
      if constexpr (MODE == EPI_SYM_DIAG) {
        // column lc + k lies above the diagonal iff k > lr - lc: take the
        // value computed at (lc + k, lr), i.e. chunk lc / 8 of column lr
        const int dd = lr - lc;
        if (dd < 7) {
          const u32x4 up = *(const __attribute__((address_space(3))) u32x4*)(Sl + stage_off(lr, lc >> 3));
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t m = (2 * w > dd ? 0x0000ffffu : 0u) | (2 * w + 1 > dd ? 0xffff0000u : 0u);
            val[w] = (val[w] & ~m) | (up[w] & m);
          }
        }
      }
      const int64_t off = lidx(e.d_pairs, m0 + lr, n0 + lc, e.ldd);
      *gmem(reinterpret_cast<u32x4*>(D + off)) = val;
      if (e.D2) {
        if constexpr (MODE == EPI_SYM_DIAG) {
          // the second output adds delta on the real diagonal, from fp32
          if (lr >= lc && lr < lc + 8 && m0 + lr < e.diag_n) {
            const int k = lr - lc;
            const uint16_t hb = __builtin_bit_cast(uint16_t, static_cast<_Float16>(fp32_value(sdiag[lr] + e.delta)));
            const uint32_t w = val[k >> 1];
            val[k >> 1] = (k & 1) ? ((w & 0xffffu) | (static_cast<uint32_t>(hb) << 16))
                                  : ((w & 0xffff0000u) | hb);
          }
        }
        *gmem(reinterpret_cast<u32x4*>(e.D2 + lidx(e.d_pairs, m0 + lr, n0 + lc, e.N))) = val;
      }
    });
  });
  // Mirror of an off-diagonal symmetric tile: row n0 + c of the output (c in
  // this wave's 64 tile columns), columns m0 + (this wave's 128 tile rows),
  // is this wave's staged column c as it stands. One instruction covers 4
  // columns x 16 chunks: in the row-pair layout, two pairs of output rows
  // over 128 columns, i.e. whole 128-byte lines (the same bytes stored
  // straight from registers would fill only half of each line they touch).
  // The 16 chunks of a column sit in one half of its swizzled slots, so a
  // column's reads hit distinct banks.
  if constexpr (MODE == EPI_SYM_OFFDIAG) {
    if (T) {
      static_for<0, Cf::WN / 4>([&](auto CB) {
        const int c = wn * Cf::WN + CB * 4 + (lane >> 4);
        const int k = wm * (Cf::WM / 8) + (lane & 15);
        const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(Sl + stage_off(c, k));
        const int64_t off = lidx(e.d_pairs, n0 + c, m0 + 8 * k, ldT);
        *gmem(reinterpret_cast<u32x4*>(T + off)) = v;
        if (T2) *gmem(reinterpret_cast<u32x4*>(T2 + off)) = v;
      });
    }
  }
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void gemm_nt_kernel(
    const GemmDesc* __restrict__ descs, int count, int total_tiles, TileDeal deal,
    int pool_begin, int* __restrict__ pool_claims) {
#if defined(__HIP_DEVICE_COMPILE__)
  // Four stages as distinct LDS objects (the loop below is unrolled by four).
  // One LDS block: during the K loop, four stages of (A slice, B slice);
  // in the epilogue, the 256 x 256 fp16 output tile (same 128 KB).
  static_assert(STAGES * (C::A_ELEMS + C::B_ELEMS) == C::BM * C::BN, "LDS reuse");
  __shared__ __attribute__((aligned(1024))) _Float16 smem[STAGES * (C::A_ELEMS + C::B_ELEMS)];
  __shared__ float sdiag[C::BM];   // fp32 diagonal of a diagonal tile (second output)
  auto stA = [&](int s) { return smem + s * (C::A_ELEMS + C::B_ELEMS); };
  auto stB = [&](int s) { return smem + s * (C::A_ELEMS + C::B_ELEMS) + C::A_ELEMS; };

  // Tiles [0, pool_begin) are dealt to the first pool_begin workgroups
  // (deal_tile); the rest form a pool that the later workgroups claim in
  // order, so the XCDs that get through their dealt tiles sooner (their
  // clocks and memory paths differ by a few per cent) take more of the pool
  // instead of waiting for the slowest at the end of the launch. The launch
  // has a few more workgroups than tiles, so that a fast XCD has claimers to
  // spare; a claimer that finds the pool empty ends at once.
  int t_logical;
  if (static_cast<int>(blockIdx.x) < pool_begin) {
    t_logical = deal_tile(blockIdx.x, pool_begin, deal);
  } else {
    __shared__ int s_claim;
    if (threadIdx.x == 0) s_claim = pool_begin + atomicAdd(pool_claims, 1);
    __syncthreads();
    t_logical = __builtin_amdgcn_readfirstlane(s_claim);
    if (t_logical >= total_tiles) return;
  }
  const int p = find_problem(descs, count, t_logical);
  const GemmDesc& d = descs[p];
  // Everything the first copies need, read here in one go (adjacent fields,
  // one batch of scalar loads and one wait) rather than one field at a time
  // at its first use.
  const _Float16* const dA = d.A;
  const _Float16* const dB = d.B;
  const int t = t_logical - d.tile_begin;
  const int tiles_n = d.tiles_n;
  const int M = d.M, N = d.N, K = d.K;
  const bool sym = d.symmetric != 0;
  const int c_is_bt = d.c_is_bt;
  const int a_pairs = d.a_pairs, b_pairs = d.b_pairs;
  const int a_kmajor = d.a_kmajor, b_kmajor = d.b_kmajor;
  const float alpha = d.alpha, beta = d.beta;
  int ti, tj;
  if (sym) decode_lower(t, tiles_n, ti, tj);
  else decode_full(t, M / C::BM, tiles_n, ti, tj);
  const int m0 = ti * C::BM, n0 = tj * C::BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  // A diagonal tile of a symmetric product computes only its stored blocks,
  // dealt out over the waves by diag_block; every element gets the same
  // arithmetic as in any other tile.
  const bool diag = sym && ti == tj;
  const int bcol0 = wn * C::WN;   // first column of this wave's blocks (other tiles)

  // beta * C taken from the B slices (C == B^T): global row i of C is
  // column k = i of B, so this wave's 32-row block I arrives with K slice
  // m0 / BK + wm * FM + I. With WM == STAGES * BK that slice sits in ring
  // position I of ring round m0 / (STAGES * BK) + wm.
  static_assert(C::FM == STAGES && C::WM == STAGES * C::BK, "fold: one ring round per wave");
  const bool fold = c_is_bt != 0 && !b_kmajor;   // the fold reads row-major B slices
  const float rho = fold ? beta / alpha : 0.f;
  const int fold_round = fold ? m0 / (STAGES * C::BK) + wm : -1;

  // zeroed once the first copies are on their way (see k_loop)
  floatx16 acc[C::FM][C::FN];
  auto zero_acc = [&]() {
    static_for<0, C::FM>([&](auto I) {
      static_for<0, C::FN>([&](auto J) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[I][J][r] = 0.f;
      });
    });
  };

  // Copies. The four waves of group 0 (tile rows 0-127) copy every A slice
  // and the four of group 1 every B slice. Each wave instruction fills 1 KB
  // of LDS = 16 tile rows of 64 bytes; lane l lands on row l/4, physical
  // chunk l%4, so it fetches logical chunk (l%4) ^ swz(row) of that row.
  // Offsets are relative to the tile's row panel; the K position goes in
  // the scalar offset: 2 bytes per column of a row-major operand, 4 in the
  // row-pair layout (a 32-column block of two rows is 128 bytes).
  // A K-major operand is copied by pairs of k rows instead (km_src): copy i
  // of wave gw fetches pair 4 gw + i of the slice, and the buffer
  // descriptor is rebased on every slice (the K offset k0 * width may
  // exceed 32 bits).
  constexpr int RPB = 1024 / (C::BK * 2);          // rows per copy instruction
  constexpr int COPIES = C::BM / RPB / C::WAVES_N; // per wave and slice
  static_assert(C::WAVES_M == 2 && COPIES == 4, "ping-pong plan: two groups of four waves");
  static_assert(C::A_ELEMS == 16 * 2 * C::BM, "K-major slice: 16 pairs of k rows per slice");
  const int grp = wm, gw = wn;
  const bool my_pairs = (grp == 0 ? a_pairs : b_pairs) != 0;
  const bool my_km = (grp == 0 ? a_kmajor : b_kmajor) != 0;
  const int64_t my_width = grp == 0 ? M : N;        // leading dimension if K-major
  const _Float16* const my_km_base = grp == 0 ? dA + 2 * static_cast<int64_t>(m0)
                                              : dB + 2 * static_cast<int64_t>(n0);
  const uint32_t panel_bytes = static_cast<uint32_t>(C::BM) * K * 2u;
  const i32x4 rMy = grp == 0 ? make_rsrc(dA + static_cast<int64_t>(m0) * K, panel_bytes)
                             : make_rsrc(dB + static_cast<int64_t>(n0) * K, panel_bytes);
  const uint32_t kbytes = my_pairs ? 4u : 2u;
  uint32_t my_off[COPIES];
  static_for<0, COPIES>([&](auto i) {
    if (my_km) {
      my_off[i] = static_cast<uint32_t>(km_src(gw * COPIES + i, lane >> 3, lane & 7, my_width)) * 2u;
    } else {
      const int row = (gw * COPIES + i) * RPB + lane / C::KCH;
      const int col = ((lane % C::KCH) ^ swz(row)) * 8;
      my_off[i] = static_cast<uint32_t>(my_pairs ? (row >> 1) * 2 * K + (row & 1) * 32 + col
                                                 : row * K + col) * 2u;
    }
  });
  // this wave's share of slice k0 of its group's operand into ring stage s
  // (KM: the operand is K-major)
  auto copy_my = [&](int s, int k0, auto KM) {
    _Float16* base = (grp == 0 ? stA(s) : stB(s)) + gw * COPIES * 512;
    if constexpr (decltype(KM)::value) {
      const i32x4 r = make_rsrc(my_km_base + static_cast<int64_t>(k0) * my_width,
                                static_cast<uint32_t>(32 * my_width * 2));
      static_for<0, COPIES>([&](auto i) {
        lds_copy16(r, lds_addr_of(base + i * 512), my_off[i], 0u);
      });
    } else {
      const uint32_t kb = static_cast<uint32_t>(k0) * kbytes;
      static_for<0, COPIES>([&](auto i) {
        lds_copy16(rMy, lds_addr_of(base + i * 512), my_off[i], kb);
      });
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // One fragment register set per wave: a wave reads the next slice's
  // fragments only in the phase after issuing its MFMAs of the current one.
  half8 fa0[C::KSTEPS][C::FM], fb0[C::KSTEPS][C::FN];
  constexpr int KM_PAIR = 2 * C::BM;   // halves per pair of k rows in a K-major slice
  auto read_frags = [&](const _Float16* SA, const _Float16* SB, auto& fa, auto& fb, auto AK,
                        auto BK) {
    static_for<0, C::KSTEPS>([&](auto KS) {
      const int kc = KS * 2 + (lane >> 5);
      static_for<0, C::FM>([&](auto I) {
        if constexpr (decltype(AK)::value) {
          fa[KS][I] = km_frag<KM_PAIR>(SA, wm * C::WM + I * 32, KS, lane);
        } else {
          const int row = wm * C::WM + I * 32 + (lane & 31);
          fa[KS][I] = *reinterpret_cast<const half8*>(&SA[row * C::BK + ((kc ^ swz(row)) * 8)]);
        }
      });
      static_for<0, C::FN>([&](auto J) {
        if constexpr (decltype(BK)::value) {
          fb[KS][J] = km_frag<KM_PAIR>(SB, bcol0 + J * 32, KS, lane);
        } else {
          const int row = bcol0 + J * 32 + (lane & 31);
          fb[KS][J] = *reinterpret_cast<const half8*>(&SB[row * C::BK + ((kc ^ swz(row)) * 8)]);
        }
      });
    });
  };
  // Diagonal-tile fragments, G = the wave's group. Group 1: A rows of blocks
  // wn .. wn + 3 in fa, of block wn + 4 in fb[.][1], B columns of block
  // column wn in fb[.][0]. Group 0: A rows of its four blocks in fa, B
  // columns of block columns wn and 7 - wn in fb[.][0] and fb[.][1].
  auto frag_at = [&](const _Float16* S, int row0, int kc) {
    const int row = row0 + (lane & 31);
    return *reinterpret_cast<const half8*>(&S[row * C::BK + ((kc ^ swz(row)) * 8)]);
  };
  auto read_frags_diag = [&](const _Float16* SA, const _Float16* SB, auto& fa, auto& fb,
                             auto G) {
    static_for<0, C::KSTEPS>([&](auto KS) {
      const int kc = KS * 2 + (lane >> 5);
      if constexpr (decltype(G)::value == 1) {
        static_for<0, 4>([&](auto B) { fa[KS][B] = frag_at(SA, (wn + B) * 32, kc); });
        fb[KS][1] = frag_at(SA, (wn + 4) * 32, kc);
        fb[KS][0] = frag_at(SB, wn * 32, kc);
      } else {
        static_for<0, 4>([&](auto B) {
          int bi, bj;
          diag_block(0, wn, B, bi, bj);
          fa[KS][B] = frag_at(SA, bi * 32, kc);
        });
        fb[KS][0] = frag_at(SB, wn * 32, kc);
        fb[KS][1] = frag_at(SB, (7 - wn) * 32, kc);
      }
    });
  };
  auto mfmas = [&](auto& fa, auto& fb) {
    static_for<0, C::KSTEPS>([&](auto KS) {
      static_for<0, C::FM>([&](auto I) {
        static_for<0, C::FN>([&](auto J) {
          acc[I][J] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[KS][I], fb[KS][J], acc[I][J],
                                                             0, 0, 0);
        });
      });
    });
  };
  // Diagonal tile: block b accumulates in acc[b % 4][b / 4]. Group 0's
  // blocks b < 3 - wn use B column wn, the others 7 - wn; the split is
  // chosen once per phase so the MFMA stream stays one straight-line block.
  auto mfmas_diag = [&](auto& fa, auto& fb, auto G) {
    if constexpr (decltype(G)::value == 1) {
      static_for<0, C::KSTEPS>([&](auto KS) {
        static_for<0, 4>([&](auto B) {
          acc[B][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[KS][B], fb[KS][0], acc[B][0],
                                                             0, 0, 0);
        });
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[KS][1], fb[KS][0], acc[0][1],
                                                           0, 0, 0);
      });
    } else {
      auto seq = [&](auto NA) {
        static_for<0, C::KSTEPS>([&](auto KS) {
          static_for<0, 4>([&](auto B) {
            constexpr int j = B < decltype(NA)::value ? 0 : 1;
            acc[B][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[KS][B], fb[KS][j], acc[B][0],
                                                               0, 0, 0);
          });
        });
      };
      if (wn == 0) seq(std::integral_constant<int, 3>{});
      else if (wn == 1) seq(std::integral_constant<int, 2>{});
      else if (wn == 2) seq(std::integral_constant<int, 1>{});
      else seq(std::integral_constant<int, 0>{});
    }
  };
  // a += rho * C for one 32 x 32 block whose rows arrive with slice SB and
  // whose columns start at col0: lane l needs rows 8g + 4(l/32) .. +3
  // (g = 0..3) of column col0 + l%32, i.e. four consecutive k of that B row,
  // 8 bytes. fold_c applies it to the wave's blocks of row block I.
  auto fold_block = [&](const _Float16* SB, int col0, floatx16& a) {
    const int row = col0 + (lane & 31);
    const _Float16* base = SB + row * C::BK + 4 * (lane >> 5);
    static_for<0, 4>([&](auto G) {
      const half4 c = *reinterpret_cast<const half4*>(base + ((G ^ swz(row)) * 8));
#pragma unroll
      for (int q = 0; q < 4; ++q)
        a[G * 4 + q] = __builtin_fmaf(rho, static_cast<float>(c[q]), a[G * 4 + q]);
    });
  };
  auto fold_c = [&](const _Float16* SB, auto I) {
    static_for<0, C::FN>([&](auto J) { fold_block(SB, bcol0 + J * 32, acc[I][J]); });
  };
  // Diagonal tile: block (bi, bj) takes beta * C from the slice holding its
  // rows, slice 8 ti + bi = ring round 2 ti + bi / 4, position bi % 4.
  auto fold_diag = [&](const _Float16* SB, auto POS, int round, auto G) {
    if (!fold || (round >> 1) != ti) return;
    constexpr int NB = decltype(G)::value == 1 ? 5 : 4;
    static_for<0, NB>([&](auto B) {
      int bi, bj;
      diag_block(decltype(G)::value, wn, B, bi, bj);
      if ((bi & 3) == decltype(POS)::value && 2 * ti + (bi >> 2) == round)
        fold_block(SB, bj * 32, acc[B % 4][B / 4]);
    });
  };
  // Ping-pong schedule, one barrier per phase. On every SIMD one wave of
  // each group is resident; in each phase one group streams MFMAs from
  // registers while the other feeds LDS:
  //   phase 2t:   group 0 multiplies slice t; group 1 copies its half of
  //               slice t+3 into the stage of slice t-1 (read by both groups
  //               by now) and reads the fragments of slice t;
  //   phase 2t+1: group 1 multiplies slice t; group 0 copies its half of
  //               slice t+4 into the stage of slice t and reads slice t+1.
  // Before each barrier a wave waits for its LDS reads and for its own
  // copies of the slice read next (at most two later slices, 8 copies,
  // stay in flight), so a slice is complete in LDS before anyone reads it.
  auto phase_end = [&]() {
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(2 * COPIES) & ~0x0F00);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // DIAG: a diagonal tile (chosen once per tile, so that the MFMA stream of
  // a phase stays one straight-line block); G: the wave's group
  auto mfma_phase = [&](auto& fa, auto& fb, auto DIAG, auto G) {
    if constexpr (decltype(DIAG)::value) mfmas_diag(fa, fb, G);
    else mfmas(fa, fb);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto read_phase = [&](const _Float16* SA, const _Float16* SB, auto& fa, auto& fb, auto DIAG,
                        auto AK, auto BK, auto G) {
    if constexpr (decltype(DIAG)::value) read_frags_diag(SA, SB, fa, fb, G);
    else read_frags(SA, SB, fa, fb, AK, BK);
  };
  // K is a multiple of STAGES * BK; requests past the last slice re-read the
  // last slice into a stage that is never consumed again.
  const int nk = K / C::BK;
  auto kclamp = [&](int sl) { return min(sl, nk - 1) * C::BK; };
  // DIAG as above; AK / BK: A / B is K-major (at most one; never with DIAG).
  // The fold is compiled only where B slices are row-major.
  auto k_loop = [&](auto DIAG, auto AK, auto BK) {
  constexpr bool IS_DIAG = decltype(DIAG)::value;
  const std::integral_constant<int, 0> G0;
  const std::integral_constant<int, 1> G1;
  constexpr bool FOLD_OK = !decltype(BK)::value;
  if (grp == 0) static_for<0, STAGES>([&](auto s) { copy_my(s, kclamp(s), AK); });
  else static_for<0, STAGES>([&](auto s) { copy_my(s, kclamp(s), BK); });
  zero_acc();
  // only slice 0 is read before the next wait; slices 1-3 keep streaming
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(3 * COPIES) & ~0x0F00);
  __builtin_amdgcn_s_barrier();
  if (grp == 0) {
    read_phase(stA(0), stB(0), fa0, fb0, DIAG, AK, BK, G0);
    if constexpr (IS_DIAG) fold_diag(stB(0), std::integral_constant<int, 0>{}, 0, G0);
    else if constexpr (FOLD_OK)
      if (fold_round == 0) fold_c(stB(0), std::integral_constant<int, 0>{});
    phase_end();
    for (int kt = 0; kt < nk; kt += STAGES) {
      static_for<0, STAGES>([&](auto U) {
        constexpr int u = U;
        auto& fa = fa0;
        auto& fb = fb0;
        auto& fan = fa0;
        auto& fbn = fb0;
        mfma_phase(fa, fb, DIAG, G0);
        phase_end();
        copy_my(u, kclamp(kt + u + 4), AK);
        read_phase(stA((u + 1) % STAGES), stB((u + 1) % STAGES), fan, fbn, DIAG, AK, BK, G0);
        if constexpr (IS_DIAG)
          fold_diag(stB((u + 1) % STAGES), std::integral_constant<int, (u + 1) % STAGES>{},
                    kt / STAGES + (u == STAGES - 1 ? 1 : 0), G0);
        else if constexpr (FOLD_OK)
          if (kt / STAGES + (u == STAGES - 1 ? 1 : 0) == fold_round)
            fold_c(stB((u + 1) % STAGES), std::integral_constant<int, (u + 1) % STAGES>{});
        phase_end();
      });
    }
  } else {
    phase_end();
    for (int kt = 0; kt < nk; kt += STAGES) {
      static_for<0, STAGES>([&](auto U) {
        constexpr int u = U;
        auto& fa = fa0;
        auto& fb = fb0;
        if (kt + u >= 1) copy_my((u + 3) % STAGES, kclamp(kt + u + 3), BK);
        read_phase(stA(u), stB(u), fa, fb, DIAG, AK, BK, G1);
        if constexpr (IS_DIAG)
          fold_diag(stB(u), std::integral_constant<int, u>{}, kt / STAGES, G1);
        else if constexpr (FOLD_OK)
          if (kt / STAGES == fold_round) fold_c(stB(u), std::integral_constant<int, u>{});
        phase_end();
        mfma_phase(fa, fb, DIAG, G1);
        phase_end();
      });
    }
  }
  };
  if (diag) k_loop(std::true_type{}, std::false_type{}, std::false_type{});
  else if (a_kmajor) k_loop(std::false_type{}, std::true_type{}, std::false_type{});
  else if (b_kmajor) k_loop(std::false_type{}, std::false_type{}, std::true_type{});
  else k_loop(std::false_type{}, std::false_type{}, std::false_type{});
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));   // trailing copies
  __builtin_amdgcn_s_barrier();

  // ---------------------------------------------------------------- epilogue
  Epi e;
  e.alpha = alpha; e.beta = beta; e.gamma = d.gamma; e.delta = d.delta;
  e.C = fold ? nullptr : d.C;   // folded C is already in the accumulators
  e.ldc = d.ldc; e.c_type = d.c_type;
  e.D = d.D; e.D2 = d.D2; e.DT = d.DT;
  e.M = M; e.N = N; e.ldd = d.ldd; e.diag_n = d.diag_n;
  e.valid_m = d.valid_m; e.valid_n = d.valid_n; e.out_type = d.out_type;
  e.c_pairs = d.c_pairs; e.d_pairs = d.d_pairs;
  e.row0 = m0 + wm * C::WM + (lane >> 5) * 4;
  e.col0 = n0 + wn * C::WN + (lane & 31);
  // The operand ring is reused as the output staging tile; all waves must
  // be done with it (and with their last fragment reads and copies).
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0) & ~0x0F00);
  __syncthreads();
  const bool row_store_ok =
      (d.ldd % 8 == 0) && (reinterpret_cast<uintptr_t>(d.D) % 16 == 0);
  if (sym) {
    if (ti != tj)
      epilogue_tile<C, EPI_SYM_OFFDIAG>(acc, e, smem, sdiag, lane, wm, wn, m0, n0,
                                        static_cast<_Float16*>(d.D), d.ldd, d.D2);
    else
      epilogue_tile<C, EPI_SYM_DIAG>(acc, e, smem, sdiag, lane, wm, wn, m0, n0, nullptr, 0,
                                     nullptr);
  } else if (d.out_type == OUT_F16 && d.valid_m == M && d.valid_n == N && row_store_ok &&
             !d.D2 && (!e.C || d.c_type == OUT_F16)) {
    if (e.C)
      epilogue_tile<C, EPI_FULL_C>(acc, e, smem, sdiag, lane, wm, wn, m0, n0, d.DT, M, nullptr);
    else
      epilogue_tile<C, EPI_FULL>(acc, e, smem, sdiag, lane, wm, wn, m0, n0, d.DT, M, nullptr);
  } else {
    epilogue_output<C>(acc, e);
  }
#endif
}
// ------------------------------------------------------------ small tiles
// The same products on 64 x 64 tiles, for stages with too few 256 x 256
// tiles to occupy the chip (a single small matrix puts one 256-tile on one
// CU per stage). Four waves, each owning one 32 x 32 block of
// v_mfma_f32_32x32x16_f16; a four-stage ring of 64 x 32 operand slices
// filled by the same buffer-to-LDS copies; per-element epilogue.
//
// K-major operands as in gemm_nt_kernel, with 64-column pairs of k rows
// (256 bytes each; one copy instruction moves four of them).
//
// Every output element is produced exactly as gemm_nt_kernel produces it:
// the same MFMA over the same 16-wide k steps in the same order, beta * C
// folded at the same K slice (before the MFMAs of the slice holding the
// element's row), the same epilogue arithmetic and the same choice of path
// (symmetric, whole-tile fp16, or clipped typed output). The two kernels
// are therefore interchangeable per stage, bit for bit.
constexpr int SM_TILE = 64;
constexpr int SM_THREADS = 256;
constexpr int SM_BK = 32;
constexpr int SM_STAGES = 4;
constexpr int SM_SLICE = SM_TILE * SM_BK;   // halves per operand slice

// Logical tile of a symmetric problem -> (ti, tj), tj <= ti, rows of the
// lower triangle in order: tile t = ti (ti + 1) / 2 + tj.
__device__ __forceinline__ void decode_lower_rows(int t, int& ti, int& tj) {
  int r = static_cast<int>((sqrtf(8.f * static_cast<float>(t) + 1.f) - 1.f) * 0.5f);
  while (r * (r + 1) / 2 > t) --r;
  while ((r + 1) * (r + 2) / 2 <= t) ++r;
  ti = r;
  tj = t - r * (r + 1) / 2;
}

template <int CT>
__device__ __forceinline__ float load_c(const GemmDesc& d, int64_t i, int64_t j) {
  return load_typed<CT>(d.C, lidx(d.c_pairs, i, j, d.ldc));
}

template <int KIND, int OT, int CT>
__device__ __forceinline__ void small_epilogue(const floatx16& acc, const GemmDesc& d, bool fold,
                                               int i0, int j0, bool diag_tile) {
  // KIND: 0 symmetric, 1 whole-tile fp16, 2 clipped typed output
  const int lane = threadIdx.x & 63;
  const int j = j0 + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = i0 + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
    if constexpr (KIND == 2) {
      if (i >= d.valid_m || j >= d.valid_n) continue;
    }
    float x = d.alpha * acc[r];
    if (!fold && d.C) {
      // the symmetric path reads C at the transposed position, as the
      // 256-tile kernel does (C is symmetric there)
      if constexpr (KIND == 2) x = __builtin_fmaf(d.beta, load_c<CT>(d, i, j), x);
      else if constexpr (KIND == 0) x = __builtin_fmaf(d.beta, load_c<OUT_F16>(d, j, i), x);
      else x = __builtin_fmaf(d.beta, load_c<OUT_F16>(d, i, j), x);
    }
    const bool on_diag = i == j && j < d.diag_n;
    if constexpr (KIND == 2) {
      if (on_diag) x += d.gamma;
      store_typed<OT>(d.D, lidx(d.d_pairs, i, j, d.ldd), fp32_value(x));
    } else {
      if (d.gamma != 0.f && on_diag) x += d.gamma;
      x = fp32_value(x);
      const _Float16 h = static_cast<_Float16>(x);
      _Float16* D = static_cast<_Float16*>(d.D);
      if constexpr (KIND == 0) {
        // lower triangle only on diagonal tiles; every stored element is
        // also stored at its mirror position, as is the second output
        if (diag_tile && j > i) continue;
        gmem(D)[lidx(d.d_pairs, i, j, d.ldd)] = h;
        gmem(D)[lidx(d.d_pairs, j, i, d.ldd)] = h;
        if (d.D2) {
          const _Float16 h2 = (i == j && i < d.diag_n)
                                  ? static_cast<_Float16>(fp32_value(x + d.delta)) : h;
          gmem(d.D2)[lidx(d.d_pairs, i, j, d.N)] = h2;
          gmem(d.D2)[lidx(d.d_pairs, j, i, d.N)] = h2;
        }
      } else {
        gmem(D)[lidx(d.d_pairs, i, j, d.ldd)] = h;
        if (d.DT) gmem(d.DT)[lidx(d.d_pairs, j, i, d.M)] = h;
      }
    }
  }
}

// KM: the launch may hold K-major operands. Stages without them use the
// KM = false kernel, whose code is a third the size: this kernel's stages
// are short, and each workgroup starts on a cold instruction cache.
template <bool KM>
__global__ __launch_bounds__(SM_THREADS) void gemm_small_kernel(
    const GemmDesc* __restrict__ descs, int count, int total_tiles) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(1024))) _Float16 smem[SM_STAGES * 2 * SM_SLICE];
  auto stA = [&](int s) { return smem + s * 2 * SM_SLICE; };
  auto stB = [&](int s) { return smem + s * 2 * SM_SLICE + SM_SLICE; };
  const int t_logical = blockIdx.x;
  const int p = find_problem(descs, count, t_logical);
  const GemmDesc& d = descs[p];
  const int t = t_logical - d.tile_begin;
  const int K = d.K;
  const bool sym = d.symmetric != 0;
  int ti, tj;
  if (sym) decode_lower_rows(t, ti, tj);
  else {
    ti = t / d.tiles_n;
    tj = t - ti * d.tiles_n;
  }
  const int m0 = ti * SM_TILE, n0 = tj * SM_TILE;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const bool fold = d.c_is_bt != 0 && !d.b_kmajor;
  const float rho = fold ? d.beta / d.alpha : 0.f;
  const int fold_slice = (m0 + 32 * wm) / SM_BK;   // this wave's rows arrive with this K slice
  floatx16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;

  // copies: wave w fills rows 16 w .. 16 w + 15 of the A and of the B slice,
  // or, for a K-major operand, pairs of k rows 4 w .. 4 w + 3 (km_src; the
  // descriptor rebased on every slice as in gemm_nt_kernel). AK / BK: A / B
  // is K-major, chosen once per tile so the loop has no per-slice branches.
  const uint32_t panel = static_cast<uint32_t>(SM_TILE) * K * 2u;
  const int nk = K / SM_BK;
  auto main_loop = [&](auto AK, auto BK) {
    constexpr bool A_KM = decltype(AK)::value, B_KM = decltype(BK)::value;
    const i32x4 rA = make_rsrc(d.A + static_cast<int64_t>(m0) * K, panel);
    const i32x4 rB = make_rsrc(d.B + static_cast<int64_t>(n0) * K, panel);
    const int row = wave * 16 + lane / 4;
    const int col = ((lane % 4) ^ swz(row)) * 8;
    const int kq = wave * 4 + (lane >> 4), ku = (lane >> 3) & 1;
    uint32_t offA, offB;
    if constexpr (A_KM) offA = static_cast<uint32_t>(km_src(kq, ku, lane & 7, d.M)) * 2u;
    else offA = static_cast<uint32_t>(d.a_pairs ? (row >> 1) * 2 * K + (row & 1) * 32 + col
                                                : row * K + col) * 2u;
    if constexpr (B_KM) offB = static_cast<uint32_t>(km_src(kq, ku, lane & 7, d.N)) * 2u;
    else offB = static_cast<uint32_t>(d.b_pairs ? (row >> 1) * 2 * K + (row & 1) * 32 + col
                                                : row * K + col) * 2u;
    const uint32_t kbA = d.a_pairs ? 4u : 2u, kbB = d.b_pairs ? 4u : 2u;
    auto copy_slice = [&](int s, int sl) {
      const uint32_t k0 = static_cast<uint32_t>(min(sl, nk - 1) * SM_BK);
      if constexpr (A_KM) {
        const i32x4 r = make_rsrc(d.A + 2 * static_cast<int64_t>(m0) + static_cast<int64_t>(k0) * d.M,
                                  static_cast<uint32_t>(32 * d.M * 2));
        lds_copy16(r, lds_addr_of(stA(s) + wave * 512), offA, 0u);
      } else {
        lds_copy16(rA, lds_addr_of(stA(s) + wave * 512), offA, k0 * kbA);
      }
      if constexpr (B_KM) {
        const i32x4 r = make_rsrc(d.B + 2 * static_cast<int64_t>(n0) + static_cast<int64_t>(k0) * d.N,
                                  static_cast<uint32_t>(32 * d.N * 2));
        lds_copy16(r, lds_addr_of(stB(s) + wave * 512), offB, 0u);
      } else {
        lds_copy16(rB, lds_addr_of(stB(s) + wave * 512), offB, k0 * kbB);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    static_for<0, SM_STAGES - 1>([&](auto s) { copy_slice(s, s); });
    half8 fa[2], fb[2];
    for (int kt = 0; kt < nk; kt += SM_STAGES) {
      static_for<0, SM_STAGES>([&](auto U) {
        constexpr int u = U;
        const int sl = kt + u;
        // own copies of slice sl done (two later slices may stay in flight),
        // then every wave's
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(4) & ~0x0F00);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        copy_slice((u + 3) % SM_STAGES, sl + 3);   // the stage of slice sl - 1, read by now
        const _Float16* SA = stA(u);
        const _Float16* SB = stB(u);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int kc = ks * 2 + (lane >> 5);
          const int ra = wm * 32 + (lane & 31), rb = wn * 32 + (lane & 31);
          if constexpr (A_KM) fa[ks] = km_frag<2 * SM_TILE>(SA, wm * 32, ks, lane);
          else fa[ks] = *reinterpret_cast<const half8*>(&SA[ra * SM_BK + ((kc ^ swz(ra)) * 8)]);
          if constexpr (B_KM) fb[ks] = km_frag<2 * SM_TILE>(SB, wn * 32, ks, lane);
          else fb[ks] = *reinterpret_cast<const half8*>(&SB[rb * SM_BK + ((kc ^ swz(rb)) * 8)]);
        }
        if constexpr (!B_KM) {
          if (fold && sl == fold_slice) {
            const int rb = wn * 32 + (lane & 31);
            const _Float16* base = SB + rb * SM_BK + 4 * (lane >> 5);
            static_for<0, 4>([&](auto G) {
              const half4 c = *reinterpret_cast<const half4*>(base + ((G ^ swz(rb)) * 8));
#pragma unroll
              for (int q = 0; q < 4; ++q)
                acc[G * 4 + q] = __builtin_fmaf(rho, static_cast<float>(c[q]), acc[G * 4 + q]);
            });
          }
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[0], fb[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[1], fb[1], acc, 0, 0, 0);
      });
    }
  };
  if constexpr (KM) {
    if (d.a_kmajor) main_loop(std::true_type{}, std::false_type{});
    else if (d.b_kmajor) main_loop(std::false_type{}, std::true_type{});
    else main_loop(std::false_type{}, std::false_type{});
  } else {
    main_loop(std::false_type{}, std::false_type{});
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));   // trailing copies

  const int i0 = m0 + wm * 32, j0 = n0 + wn * 32;
  // the path gemm_nt_kernel takes for this descriptor
  const bool row_store_ok =
      (d.ldd % 8 == 0) && (reinterpret_cast<uintptr_t>(d.D) % 16 == 0);
  const bool c_unfolded_f16 = fold || !d.C || d.c_type == OUT_F16;
  if (sym) {
    small_epilogue<0, OUT_F16, OUT_F16>(acc, d, fold, i0, j0, ti == tj);
  } else if (d.out_type == OUT_F16 && d.valid_m == d.M && d.valid_n == d.N && row_store_ok &&
             !d.D2 && c_unfolded_f16) {
    small_epilogue<1, OUT_F16, OUT_F16>(acc, d, fold, i0, j0, false);
  } else {
    const int ct = (fold || !d.C) ? -1 : d.c_type;
#define NSMI_SMALL_OUT(OT)                                                            \
    if (d.out_type == OT) {                                                          \
      if (ct == OUT_F16) small_epilogue<2, OT, OUT_F16>(acc, d, fold, i0, j0, false); \
      else if (ct == OUT_F32) small_epilogue<2, OT, OUT_F32>(acc, d, fold, i0, j0, false); \
      else if (ct == OUT_BF16) small_epilogue<2, OT, OUT_BF16>(acc, d, fold, i0, j0, false); \
      else small_epilogue<2, OT, -1>(acc, d, fold, i0, j0, false);                     \
    }
    NSMI_SMALL_OUT(OUT_F16)
    NSMI_SMALL_OUT(OUT_F32)
    NSMI_SMALL_OUT(OUT_BF16)
#undef NSMI_SMALL_OUT
  }
#endif
}

}  // namespace

int gemm_tile() { return MainCfg::BM; }
int gemm_k_multiple() { return STAGES * MainCfg::BK; }

int gemm_small_tile() { return SM_TILE; }

hipError_t launch_gemm_small(const GemmDesc* descs, int count, int total_tiles, bool kmajor,
                             hipStream_t stream) {
  if (total_tiles <= 0 || count <= 0) return hipSuccess;
  if (kmajor)
    hipLaunchKernelGGL(gemm_small_kernel<true>, dim3(total_tiles), dim3(SM_THREADS), 0, stream,
                       descs, count, total_tiles);
  else
    hipLaunchKernelGGL(gemm_small_kernel<false>, dim3(total_tiles), dim3(SM_THREADS), 0, stream,
                       descs, count, total_tiles);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmDesc* descs, int count, int total_tiles, const GemmCtl& ctl,
                       int* pool_claims, hipStream_t stream) {
  if (total_tiles <= 0 || count <= 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_nt_kernel<MainCfg>, dim3(total_tiles + ctl.surplus),
                     dim3(MainCfg::THREADS), 0, stream, descs, count, total_tiles, ctl.deal,
                     ctl.pool_begin, pool_claims);
  return hipGetLastError();
}

}  // namespace nsmi
