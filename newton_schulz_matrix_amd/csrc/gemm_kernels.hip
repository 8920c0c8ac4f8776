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
// then mirrored), so a symmetric right operand B equals B^T; and the
// iteration keeps X^T next to X so that Q X = Q (X^T)^T is NT as well.
//
// Uses on the "Newton-Schulz 变体" page: the Gram product R = X X^T
// (section "Gram 空间 NS", SYRK: lower-triangle tiles only, about half the
// tiles), Z = b R + c R^2 (equation Z_k, epilogue alpha = c, beta = b,
// C = R, plus the fused Q = Z + a I output on the first step after a start
// or restart), Q <- Z Q + a Q (equation Q_{k+1}), the R recurrence
// T = Z R + a R, R <- T Z + a T, the restart and output products Q X, and
// the direct-space step X <- a X + (b A + c A^2) X (section "直接空间 NS").
//
// Kernel structure: BM x BN x BK workgroup tile, waves of 64 lanes each
// owning a WM x WN sub-tile built from 32x32x16 fp16 MFMAs; A and B tiles
// double-buffered in LDS with an XOR swizzle of the 16-byte chunks (so the
// 128-bit fragment reads of 8 consecutive rows hit distinct banks); global
// loads of tile k+1 issued before the MFMAs of tile k. Workgroup ids are
// remapped so each XCD (8 per MI355X, one L2 each) works on runs of 32
// neighbouring tiles, which share operand panels in its L2.
#include "ns_internal.h"

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
  static constexpr int A_LOADS = BM * KCH / THREADS;
  static constexpr int B_LOADS = BN * KCH / THREADS;
  static constexpr int KSTEPS = BK / 16;
  static constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK;
  static_assert(BM == BN, "square tiles (symmetric mode mirrors tiles)");
  static_assert(KCH == 8, "swizzle assumes 8 chunks per row");
  static_assert(A_LOADS * THREADS == BM * KCH, "A tile / thread mismatch");
  static_assert(B_LOADS * THREADS == BN * KCH, "B tile / thread mismatch");
};

using MainCfg = Cfg<128, 128, 64, 64, 64>;

// Workgroup id -> logical tile. Hardware hands workgroups to the 8 XCDs
// round-robin (id % 8). Logical tiles are cut into chunks of 32; chunk c
// goes to XCD c % 8, so each XCD walks its own run of 32 consecutive
// logical tiles while the global order of chunks (largest problems first)
// is kept. Identity on the ragged tail beyond the last multiple of 256.
__device__ __forceinline__ int xcd_remap(int wg, int total) {
  const int full = (total / 256) * 256;
  if (wg >= full) return wg;
  const int xcd = wg & 7, j = wg >> 3;
  const int chunk = (j >> 5) * 8 + xcd;
  return chunk * 32 + (j & 31);
}

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

// Logical tile of a symmetric problem -> (ti, tj), tj <= ti, row by row.
__device__ __forceinline__ void decode_lower(int t, int& ti, int& tj) {
  int r = static_cast<int>((sqrtf(8.f * t + 1.f) - 1.f) * 0.5f);
  while ((r + 1) * (r + 2) / 2 <= t) ++r;
  while (r * (r + 1) / 2 > t) --r;
  ti = r;
  tj = t - r * (r + 1) / 2;
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

__device__ __forceinline__ void store_out(void* D, int out_type, int64_t idx, float v) {
  if (out_type == OUT_F16) {
    gmem(static_cast<_Float16*>(D))[idx] = static_cast<_Float16>(v);
  } else if (out_type == OUT_F32) {
    gmem(static_cast<float*>(D))[idx] = v;
  } else {
    gmem(static_cast<uint16_t*>(D))[idx] = to_bf16_bits(v);
  }
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void gemm_nt_kernel(
    const GemmDesc* __restrict__ descs, int count, int total_tiles) {
  __shared__ __attribute__((aligned(16))) _Float16 sA[2][C::A_ELEMS];
  __shared__ __attribute__((aligned(16))) _Float16 sB[2][C::B_ELEMS];

  const int t_logical = xcd_remap(blockIdx.x, total_tiles);
  const int p = find_problem(descs, count, t_logical);
  const GemmDesc& d = descs[p];
  const int t = t_logical - d.tile_begin;
  const int M = d.M, N = d.N, K = d.K;
  const bool sym = d.symmetric != 0;
  int ti, tj;
  if (sym) decode_lower(t, ti, tj);
  else decode_full(t, M / C::BM, d.tiles_n, ti, tj);
  const int m0 = ti * C::BM, n0 = tj * C::BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

  // Buffer resources over this tile's A and B row panels: loads use 32-bit
  // offsets from a scalar base, and anything past the panel reads as zero.
  const uint32_t panel_bytes = static_cast<uint32_t>(C::BM) * K * 2u;
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<_Float16*>(d.A + static_cast<int64_t>(m0) * K), (short)0, panel_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<_Float16*>(d.B + static_cast<int64_t>(n0) * K), (short)0, panel_bytes, 0x00020000);

  floatx16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Per-thread 16-byte chunks of the A and B tiles: byte offset inside the
  // panel (at k0 = 0) and LDS element offset (XOR-swizzled chunk).
  uint32_t a_goff[C::A_LOADS], b_goff[C::B_LOADS];
  int a_soff[C::A_LOADS], b_soff[C::B_LOADS];
#pragma unroll
  for (int l = 0; l < C::A_LOADS; ++l) {
    const int c = tid + l * C::THREADS;
    const int row = c / C::KCH, kc = c % C::KCH;
    a_goff[l] = (static_cast<uint32_t>(row) * K + kc * 8) * 2u;
    a_soff[l] = row * C::BK + ((kc ^ (row & 7)) * 8);
  }
#pragma unroll
  for (int l = 0; l < C::B_LOADS; ++l) {
    const int c = tid + l * C::THREADS;
    const int row = c / C::KCH, kc = c % C::KCH;
    b_goff[l] = (static_cast<uint32_t>(row) * K + kc * 8) * 2u;
    b_soff[l] = row * C::BK + ((kc ^ (row & 7)) * 8);
  }
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 ra[C::A_LOADS], rb[C::B_LOADS];
#define NSMI_GLOAD(k0)                                                               \
  do {                                                                               \
    const int kb_ = (k0) * 2;                                                        \
    _Pragma("unroll") for (int l = 0; l < C::A_LOADS; ++l) ra[l] =                   \
        __builtin_amdgcn_raw_buffer_load_b128(rA, a_goff[l], kb_, 0);                \
    _Pragma("unroll") for (int l = 0; l < C::B_LOADS; ++l) rb[l] =                   \
        __builtin_amdgcn_raw_buffer_load_b128(rB, b_goff[l], kb_, 0);                \
  } while (0)
#define NSMI_SSTORE(s)                                                               \
  do {                                                                               \
    _Pragma("unroll") for (int l = 0; l < C::A_LOADS; ++l)                           \
        *reinterpret_cast<u32x4*>(&sA[s][a_soff[l]]) = ra[l];                        \
    _Pragma("unroll") for (int l = 0; l < C::B_LOADS; ++l)                           \
        *reinterpret_cast<u32x4*>(&sB[s][b_soff[l]]) = rb[l];                        \
  } while (0)

  const int nk = K / C::BK;
  NSMI_GLOAD(0);
  NSMI_SSTORE(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    // prefetch the next K tile (the last iteration re-reads its own tile,
    // which keeps the loop free of branches around the loads)
    NSMI_GLOAD(min(kt + 1, nk - 1) * C::BK);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      const int kc = ks * 2 + (lane >> 5);
      half8 af[C::FM], bf[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int row = wm * C::WM + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const half8*>(&sA[cur][row * C::BK + ((kc ^ (row & 7)) * 8)]);
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int row = wn * C::WN + j * 32 + (lane & 31);
        bf[j] = *reinterpret_cast<const half8*>(&sB[cur][row * C::BK + ((kc ^ (row & 7)) * 8)]);
      }
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    NSMI_SSTORE(cur ^ 1);
    __syncthreads();
  }
#undef NSMI_GLOAD
#undef NSMI_SSTORE

  // ---------------------------------------------------------------- epilogue
  // MFMA 32x32 output layout: register r of lane l holds row
  // 8*(r/4) + 4*(l/32) + r%4 and column l%32 of the 32x32 block.
  const float alpha = d.alpha, beta = d.beta, gamma = d.gamma, delta = d.delta;
  const _Float16* Cg = d.C;
  void* Dg = d.D;
  _Float16* D2g = d.D2;
  _Float16* DTg = d.DT;
  const int ldd = d.ldd, diag_n = d.diag_n;
  const int valid_m = d.valid_m, valid_n = d.valid_n, out_type = d.out_type;
  const bool diag_tile = sym && (ti == tj);

#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int col = n0 + wn * C::WN + j * 32 + (lane & 31);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int rb0 = m0 + wm * C::WM + i * 32 + g * 8 + (lane >> 5) * 4;
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = rb0 + q;
          float x = alpha * acc[i][j][g * 4 + q];
          if (Cg) x += beta * static_cast<float>(gmem(Cg)[static_cast<int64_t>(row) * N + col]);
          if (row == col && row < diag_n) x += gamma;
          v[q] = x;
        }
        if (sym) {
          // lower-triangle element (row >= col) stored at (row, col) and
          // mirrored to (col, row)
          if (diag_tile) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int row = rb0 + q;
              if (row < col) continue;
              const _Float16 h = static_cast<_Float16>(v[q]);
              gmem(static_cast<_Float16*>(Dg))[static_cast<int64_t>(row) * ldd + col] = h;
              if (row != col) gmem(static_cast<_Float16*>(Dg))[static_cast<int64_t>(col) * ldd + row] = h;
              if (D2g) {
                const float y = v[q] + ((row == col && row < diag_n) ? delta : 0.f);
                const _Float16 h2 = static_cast<_Float16>(y);
                gmem(D2g)[static_cast<int64_t>(row) * N + col] = h2;
                if (row != col) gmem(D2g)[static_cast<int64_t>(col) * N + row] = h2;
              }
            }
          } else {
            half4 hv;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              hv[q] = static_cast<_Float16>(v[q]);
              gmem(static_cast<_Float16*>(Dg))[static_cast<int64_t>(rb0 + q) * ldd + col] = hv[q];
            }
            *gmem(reinterpret_cast<half4*>(static_cast<_Float16*>(Dg) + static_cast<int64_t>(col) * ldd + rb0)) = hv;
            if (D2g) {
#pragma unroll
              for (int q = 0; q < 4; ++q) gmem(D2g)[static_cast<int64_t>(rb0 + q) * N + col] = hv[q];
              *gmem(reinterpret_cast<half4*>(D2g + static_cast<int64_t>(col) * N + rb0)) = hv;
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = rb0 + q;
            if (row < valid_m && col < valid_n)
              store_out(Dg, out_type, static_cast<int64_t>(row) * ldd + col, v[q]);
          }
          if (D2g) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int row = rb0 + q;
              const float y = v[q] + ((row == col && row < diag_n) ? delta : 0.f);
              gmem(D2g)[static_cast<int64_t>(row) * N + col] = static_cast<_Float16>(y);
            }
          }
          if (DTg) {
            half4 hv;
#pragma unroll
            for (int q = 0; q < 4; ++q) hv[q] = static_cast<_Float16>(v[q]);
            *gmem(reinterpret_cast<half4*>(DTg + static_cast<int64_t>(col) * M + rb0)) = hv;
          }
        }
      }
    }
  }
}

}  // namespace

int gemm_tile() { return MainCfg::BM; }

hipError_t launch_gemm(const GemmDesc* descs, int count, int total_tiles,
                       hipStream_t stream) {
  if (total_tiles <= 0 || count <= 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_nt_kernel<MainCfg>, dim3(total_tiles), dim3(MainCfg::THREADS),
                     0, stream, descs, count, total_tiles);
  return hipGetLastError();
}

}  // namespace nsmi
