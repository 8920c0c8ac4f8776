// Precision pipeline, steps 1 and 2 ("Newton-Schulz 变体" page, section
// "精度流水线"): X = fp16(G / (||G||_F + eps)), the norm accumulated in fp32.
//
// Three launches, each over all matrices of a call:
//   sumsq     one workgroup per SQ_ROWS x SQ_COLS chunk: fp32 sum of squares
//             of the upcast input, reduced across the wavefront with
//             butterfly shuffles and across waves in LDS (fixed order);
//   finalize  one workgroup per matrix: fixed-order sum of its chunk
//             partials, then sqrt;
//   cast      one workgroup per 64 x 64 tile of the zero-padded output: the
//             quotient rounded to nearest-even fp16, written row-major and,
//             through an LDS transpose, transposed.
// The pass is HBM-bound: it reads G twice (sumsq, cast) and writes two fp16
// copies of it.
#include "ns_internal.h"

namespace nsmi {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Load 8 consecutive elements (row `row`, columns col .. col+7) of a
// row-major matrix of type `type`, m x n, leading dimension ld, as fp32.
// Elements outside [0, m) x [0, n) read as 0.
__device__ __forceinline__ void load8p(const void* base, int type, int64_t ld, int m, int n,
                                       bool vec_ok, int row, int col, float (&v)[8]) {
  if (row >= m) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
    return;
  }
  const int64_t off = static_cast<int64_t>(row) * ld + col;
  if (vec_ok && col + 8 <= n) {
    if (type == OUT_F32) {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
      const float4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
      const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t lo = static_cast<uint16_t>(w[e] & 0xffffu);
        const uint16_t hi = static_cast<uint16_t>(w[e] >> 16);
        if (type == OUT_BF16) {
          v[2 * e] = bf16_to_f32(lo);
          v[2 * e + 1] = bf16_to_f32(hi);
        } else {
          v[2 * e] = static_cast<float>(__builtin_bit_cast(_Float16, lo));
          v[2 * e + 1] = static_cast<float>(__builtin_bit_cast(_Float16, hi));
        }
      }
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = col + e;
    float x = 0.f;
    if (c < n) {
      if (type == OUT_F32) {
        x = static_cast<const float*>(base)[off + e];
      } else {
        const uint16_t b = static_cast<const uint16_t*>(base)[off + e];
        x = type == OUT_BF16 ? bf16_to_f32(b)
                             : static_cast<float>(__builtin_bit_cast(_Float16, b));
      }
    }
    v[e] = x;
  }
}

__device__ __forceinline__ void load8(const NormDesc& d, bool vec_ok, int row, int col,
                                      float (&v)[8]) {
  load8p(d.G, d.g_type, d.ldg, d.m, d.n, vec_ok, row, col, v);
}

// Round to the storage type (nearest even) and back to fp32.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Store 8 fp32 values to row `row`, columns col .. col+7 (clipped to
// [0, m) x [0, n)) of a row-major matrix of type `type`, rounding each to
// nearest even; v is replaced by the stored (rounded) values.
__device__ __forceinline__ void store8p(void* base, int type, int64_t ld, int m, int n,
                                        bool vec_ok, int row, int col, float (&v)[8]) {
  const int64_t off = static_cast<int64_t>(row) * ld + col;
  uint16_t bits[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (type == OUT_F32) continue;
    if (type == OUT_BF16) {
      bits[e] = f32_to_bf16_bits(v[e]);
      v[e] = bf16_to_f32(bits[e]);
    } else {
      const _Float16 hv = static_cast<_Float16>(v[e]);
      bits[e] = __builtin_bit_cast(uint16_t, hv);
      v[e] = static_cast<float>(hv);
    }
  }
  if (row >= m) return;
  if (vec_ok && col + 8 <= n) {   // 16-byte aligned row piece
    if (type == OUT_F32) {
      float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + off);
      p[0] = make_float4(v[0], v[1], v[2], v[3]);
      p[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
      uint4 w;
      __builtin_memcpy(&w, bits, 16);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off) = w;
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (col + e >= n) continue;
    if (type == OUT_F32) static_cast<float*>(base)[off + e] = v[e];
    else if (type == OUT_BF16) static_cast<uint16_t*>(base)[off + e] = f32_to_bf16_bits(v[e]);
    else static_cast<_Float16*>(base)[off + e] = static_cast<_Float16>(v[e]);
  }
}

__device__ __forceinline__ bool vector_ok(const NormDesc& d) {
  const int elem = d.g_type == OUT_F32 ? 4 : 2;
  const int per16 = 16 / elem;
  return (reinterpret_cast<uintptr_t>(d.G) % 16 == 0) && (d.ldg % per16 == 0);
}

// Index of the descriptor whose [begin, begin + n) range holds `x`.
template <class F>
__device__ __forceinline__ int find_desc(int count, int x, F begin_of) {
  int lo = 0, hi = count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (begin_of(mid) <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Deterministic sum over a 256-thread block (4 waves of 64).
__device__ __forceinline__ float block_sum256(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
  if (threadIdx.x == 0) t = (red[0] + red[1]) + (red[2] + red[3]);
  return t;  // valid in thread 0 only
}

__global__ __launch_bounds__(256) void sumsq_kernel(const NormDesc* __restrict__ descs,
                                                    int count) {
  __shared__ float red[4];
  const int chunk = blockIdx.x;
  const int p = find_desc(count, chunk, [&](int i) { return descs[i].chunk_begin; });
  const NormDesc d = descs[p];
  const int c = chunk - d.chunk_begin;
  const int cr = c / d.chunks_n, cc = c - cr * d.chunks_n;
  const int col = cc * SQ_COLS + (threadIdx.x & 31) * 8;
  const int row0 = cr * SQ_ROWS + (threadIdx.x >> 5);
  const bool vec = vector_ok(d);
  float acc = 0.f;
  if (!d.grad) {
#pragma unroll
    for (int q = 0; q < SQ_ROWS / 8; ++q) {
      float v[8];
      load8(d, vec, row0 + 8 * q, col, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(v[e], v[e], acc);
    }
  } else {
    // momentum step: each element read and written by this thread only
    const int ge = d.grad_type == OUT_F32 ? 4 : 2;
    const bool gvec = (reinterpret_cast<uintptr_t>(d.grad) % 16 == 0) && (d.ldgrad % (16 / ge) == 0);
#pragma unroll
    for (int q = 0; q < SQ_ROWS / 8; ++q) {
      const int row = row0 + 8 * q;
      float v[8], g[8];
      load8(d, vec, row, col, v);
      load8p(d.grad, d.grad_type, d.ldgrad, d.m, d.n, gvec, row, col, g);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = fmaf(d.beta, v[e], g[e]);
      store8p(const_cast<void*>(d.G), d.g_type, d.ldg, d.m, d.n, vec, row, col, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(v[e], v[e], acc);
    }
  }
  const float s = block_sum256(acc, red);
  if (threadIdx.x == 0) d.partials[d.chunk_begin + c] = s;
}

__global__ __launch_bounds__(256) void finalize_kernel(const NormDesc* __restrict__ descs) {
  __shared__ float red[4];
  const NormDesc d = descs[blockIdx.x];
  float acc = 0.f;
  for (int i = threadIdx.x; i < d.chunks; i += 256) acc += d.partials[d.chunk_begin + i];
  const float s = block_sum256(acc, red);
  if (threadIdx.x == 0) {
    const float nrm = sqrtf(s);
    *d.norm_slot = nrm;
    if (d.norm_out) *d.norm_out = nrm;
  }
}

__global__ __launch_bounds__(256) void cast_kernel(const NormDesc* __restrict__ descs,
                                                   int count) {
  __shared__ _Float16 tile[CAST_TILE][CAST_TILE + 8];
  const int b = blockIdx.x;
  const int p = find_desc(count, b, [&](int i) { return descs[i].tile_begin; });
  const NormDesc d = descs[p];
  const int t = b - d.tile_begin;
  const int ti = t / d.tiles_n, tj = t - ti * d.tiles_n;
  const int i0 = ti * CAST_TILE, j0 = tj * CAST_TILE;
  const float denom = *d.norm_slot + d.eps;
  const bool vec = vector_ok(d);
  const int c8 = (threadIdx.x & 7) * 8;
  const int r = threadIdx.x >> 3;  // 0..31

#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int li = r + 32 * q;
    const int i = i0 + li, j = j0 + c8;
    float v[8];
    load8(d, vec, i, j, v);
    _Float16 h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h[e] = static_cast<_Float16>(v[e] / denom);
      tile[li][c8 + e] = h[e];
    }
    if (d.P && i < d.pm) {
      _Float16* dst = d.P + (d.pairs ? pair_index(i, j, d.ldp) : static_cast<int64_t>(i) * d.ldp + j);
      if (j + 8 <= d.pn && (reinterpret_cast<uintptr_t>(dst) % 16 == 0)) {
        uint4 w;
        __builtin_memcpy(&w, h, 16);
        *reinterpret_cast<uint4*>(dst) = w;
      } else {
        for (int e = 0; e < 8; ++e)
          if (j + e < d.pn) dst[e] = h[e];
      }
    }
  }
  if (!d.PT) return;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int lj = r + 32 * q;            // row of PT inside the tile
    const int jrow = j0 + lj, icol = i0 + c8;
    if (jrow >= d.pn) continue;
    _Float16 h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = tile[c8 + e][lj];
    _Float16* dst =
        d.PT + (d.pairs ? pair_index(jrow, icol, d.ldpt) : static_cast<int64_t>(jrow) * d.ldpt + icol);
    if (icol + 8 <= d.pm && (reinterpret_cast<uintptr_t>(dst) % 16 == 0)) {
      uint4 w;
      __builtin_memcpy(&w, h, 16);
      *reinterpret_cast<uint4*>(dst) = w;
    } else {
      for (int e = 0; e < 8; ++e)
        if (icol + e < d.pm) dst[e] = h[e];
    }
  }
}

// Shard reduction: each thread sums 8 consecutive elements of every part
// in index order (fp32), rounds once and stores 16 bytes.
__global__ __launch_bounds__(256) void reduce_kernel(const ReduceDesc* __restrict__ descs,
                                                     int count) {
  const int b = blockIdx.x;
  const int p = find_desc(count, b, [&](int i) { return descs[i].block_begin; });
  const ReduceDesc& d = descs[p];
  const int64_t i0 = static_cast<int64_t>(b - d.block_begin) * REDUCE_ELEMS + threadIdx.x * 8;
  if (i0 >= d.elems) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < d.count; ++k) {
    uint4 w = *reinterpret_cast<const uint4*>(d.parts[k] + i0);
    _Float16 h[8];
    __builtin_memcpy(h, &w, 16);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += static_cast<float>(h[e]);
  }
  _Float16 o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = static_cast<_Float16>(acc[e]);
  uint4 w;
  __builtin_memcpy(&w, o, 16);
  *reinterpret_cast<uint4*>(d.out + i0) = w;
}

// Descriptor table upload: `bytes` (a multiple of 16, at most TABLE_CHUNK)
// from the kernel argument to dst, 16 bytes per thread.
__global__ __launch_bounds__(128) void table_fill_kernel(unsigned char* __restrict__ dst,
                                                         TableChunk chunk, int bytes) {
  const int i = threadIdx.x * 16;
  if (i < bytes) {
    uint4 w;
    __builtin_memcpy(&w, chunk.bytes + i, 16);
    *reinterpret_cast<uint4*>(dst + i) = w;
  }
}

}  // namespace

hipError_t launch_table_fill(unsigned char* dst, const TableChunk& chunk, int bytes,
                             hipStream_t stream) {
  static_assert(TABLE_CHUNK == 128 * 16, "one 16-byte piece per thread");
  if (bytes <= 0) return hipSuccess;
  hipLaunchKernelGGL(table_fill_kernel, dim3(1), dim3(128), 0, stream, dst, chunk, bytes);
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceDesc* descs, int count, int total_blocks,
                         hipStream_t stream) {
  if (total_blocks <= 0 || count <= 0) return hipSuccess;
  hipLaunchKernelGGL(reduce_kernel, dim3(total_blocks), dim3(256), 0, stream, descs, count);
  return hipGetLastError();
}

hipError_t launch_sumsq(const NormDesc* descs, int count, int total_chunks,
                        hipStream_t stream) {
  if (total_chunks <= 0) return hipSuccess;
  hipLaunchKernelGGL(sumsq_kernel, dim3(total_chunks), dim3(256), 0, stream, descs, count);
  return hipGetLastError();
}

hipError_t launch_norm_finalize(const NormDesc* descs, int count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(finalize_kernel, dim3(count), dim3(256), 0, stream, descs);
  return hipGetLastError();
}

hipError_t launch_cast(const NormDesc* descs, int count, int total_tiles,
                       hipStream_t stream) {
  if (total_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(cast_kernel, dim3(total_tiles), dim3(256), 0, stream, descs, count);
  return hipGetLastError();
}

}  // namespace nsmi
