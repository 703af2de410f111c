// kvepi_ceiling.hip -- reference memory kernels for measuring what the
// epilog's launches could reach on this device (libkvepi_ceiling.so; used by
// bench.py, not part of the epilog's C ABI).
//
// The epilog moves bytes and nothing else limits it, so its fraction of the
// 8 TB/s peak is compared with plain kernels timed in the same run:
//  - kvc_stream: a streaming kernel that reads R and writes W 1-KiB wave
//    segments per step (R:W = 1:1 is a copy, 1:0 read-only, 2:1 close to the
//    fused d = 576 workload's 1408:672, 4:1 to the d = 128 indexer's 256:68),
//    every access a 16-byte nontemporal load or a plain 16-byte store;
//  - kvc_scatter_rows: the epilog's own memory pattern with no arithmetic --
//    for each token with a valid slot, read its src row (contiguous rows of
//    src_row_bytes) and write row_bytes to the slot's row of a paged cache
//    (block size, row pitch and block stride as the epilog's cache);
//  - kvc_empty: an empty kernel with a given grid (the launch floor);
//  - kvc_clock: the shader clock, from one wave that reads the core clock
//    counter and the constant 100 MHz counter around a dependent FMA chain.
//
// Exported functions (plain pointers and sizes; 0 on success, otherwise the
// hipError_t of the launch):
//   int kvc_stream(const void *src, void *dst, void *sink, uint64_t steps,
//                  int32_t r, int32_t w, int32_t blocks, void *stream);
//     src holds steps * r KiB, dst steps * w KiB (both 16-byte aligned);
//     sink holds 16 bytes per thread of the grid (blocks * 256 * 16 bytes);
//     (r, w) in {(1,0), (0,1), (1,1), (2,1), (4,1)}; blocks >= 1.
//   int kvc_scatter_rows(const void *src, int64_t src_pitch, int32_t src_row_bytes,
//                        const int32_t *slots, int32_t n_rows, void *dst,
//                        int32_t row_bytes, int32_t block_size, int64_t dst_pitch,
//                        int64_t block_stride, int32_t num_slots, int32_t blocks,
//                        void *stream);
//     byte sizes; src_row_bytes, row_bytes, src_pitch, dst_pitch and
//     block_stride multiples of 16 and src / dst 16-byte aligned; rows of
//     up to 2 KiB (32 lanes x 4 pieces of 16 bytes; rows of up to 256
//     bytes on 16 lanes, four rows per wave step); slots outside
//     [0, num_slots) skip the row.
//   int kvc_empty(int32_t blocks, void *stream);
//   int kvc_clock(uint64_t *out, int32_t spins, void *stream);
//     out: DEVICE, 4 uint64 (core clock before / after, 100 MHz counter
//     before / after); the clock in MHz is 100 * dcore / dref.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4_t ld_nt(const u32x4_t *p) { return __builtin_nontemporal_load(p); }

// Step s reads the R KiB at src + s * R KiB and writes the W KiB at
// dst + s * W KiB; each wave takes steps wave, wave + nwaves, ..., U at a
// time (all their loads issued before their stores).  Written chunk j of a
// step is the XOR of its loads j, j + W, ...; with W = 0 the loads are folded
// into the sink.
template <int R, int W, int U>
__global__ __launch_bounds__(256) void stream_kernel(const u32x4_t *__restrict__ src,
                                                     u32x4_t *__restrict__ dst,
                                                     u32x4_t *__restrict__ sink,
                                                     uint64_t steps) {
  const int lane = threadIdx.x & 63;
  const uint64_t wave = (uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const uint64_t nwaves = (uint64_t)gridDim.x * 4;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (uint64_t s0 = wave; s0 < steps; s0 += U * nwaves) {
    u32x4_t v[U][R > 0 ? R : 1];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t s = s0 + (uint64_t)u * nwaves;
#pragma unroll
      for (int r = 0; r < R; ++r)
        v[u][r] = s < steps ? ld_nt(src + (s * R + r) * 64 + lane) : acc;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t s = s0 + (uint64_t)u * nwaves;
      if constexpr (W == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) acc ^= v[u][r];
      } else {
        u32x4_t o[W];
#pragma unroll
        for (int w = 0; w < W; ++w) o[w] = (u32x4_t){0u, 0u, 0u, 0u};
#pragma unroll
        for (int r = 0; r < R; ++r) o[r % W] ^= v[u][r];
        if (s < steps) {
#pragma unroll
          for (int w = 0; w < W; ++w) dst[(s * W + w) * 64 + lane] = o[w];
        }
      }
    }
  }
  if constexpr (W == 0) sink[(uint64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// The epilog's memory pattern: a wave takes 64 / LR rows per step (lanes
// LR*i .. LR*i + LR-1 row RPS*g + i), as the epilog lays its rows out (32
// lanes a row, or 16 for rows of up to 256 bytes), reads each live row's src
// bytes with 16-byte loads (KP per lane) and writes row_bytes to its slot's
// cache row with 16-byte stores; the steps of a wave are nwaves apart, two of
// them in flight (the loads of both issued before the stores of either).  A
// lane's read pieces past the written ones are folded into its first written
// piece.  (A lane that writes no piece of a row still issues its loads: their
// use depends on the row widths, which the compiler does not know.  An
// accumulator of those loads cost the 32-lane form 5 VGPRs and a wave per
// SIMD.)
template <int LR, int KP>
__global__ __launch_bounds__(256) void scatter_kernel(const uint8_t *__restrict__ src,
                                                      int64_t src_pitch, int32_t src_row_bytes,
                                                      const int32_t *__restrict__ slots,
                                                      int32_t n_rows, uint8_t *__restrict__ dst,
                                                      int32_t row_bytes, int32_t block_size,
                                                      int64_t dst_pitch, int64_t block_stride,
                                                      int32_t num_slots) {
  constexpr int U = 2, RPS = 64 / LR;
  const int lane = threadIdx.x & 63;
  const int sub = lane / LR, li = lane % LR;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const int64_t n_steps = ((int64_t)n_rows + RPS - 1) / RPS;
  const int rp = src_row_bytes / 16, wp = row_bytes / 16;
  for (int64_t g0 = wave; g0 < n_steps; g0 += U * nwaves) {
    int32_t s[U];
    bool live[U];
    u32x4_t v[U][KP];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = RPS * (g0 + u * nwaves) + sub;
      s[u] = row < n_rows ? __builtin_nontemporal_load(slots + row) : -1;
      live[u] = s[u] >= 0 && s[u] < num_slots;
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        const int p = li + LR * k;
        v[u][k] = (live[u] && p < rp)
                      ? ld_nt(reinterpret_cast<const u32x4_t *>(src + row * src_pitch + 16 * p))
                      : (u32x4_t){0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!live[u]) continue;
      uint8_t *d = dst + (int64_t)(s[u] / block_size) * block_stride +
                   (int64_t)(s[u] % block_size) * dst_pitch;
      u32x4_t extra = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int k = 0; k < KP; ++k)
        if (li + LR * k >= wp) extra ^= v[u][k];
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        const int p = li + LR * k;
        if (p < wp)
          *reinterpret_cast<u32x4_t *>(d + 16 * p) = k == 0 ? v[u][k] ^ extra : v[u][k];
      }
    }
  }
}

__global__ void empty_kernel() {}

__global__ void clock_kernel(unsigned long long *out, int spins) {
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  float x = 1.0f + (float)threadIdx.x;
  for (int i = 0; i < spins; ++i) x = __builtin_fmaf(x, 0.999f, 0.5f);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[0] = t0;
    out[1] = t1;
    out[2] = r0;
    out[3] = x == 0.0f ? 0ull : r1;  // (x keeps the chain live)
  }
}

template <int R, int W>
hipError_t launch_stream(const void *src, void *dst, void *sink, uint64_t steps, int blocks,
                         hipStream_t st) {
  hipLaunchKernelGGL((stream_kernel<R, W, 2>), dim3(blocks), dim3(256), 0, st,
                     static_cast<const u32x4_t *>(src), static_cast<u32x4_t *>(dst),
                     static_cast<u32x4_t *>(sink), steps);
  return hipGetLastError();
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int kvc_stream(const void *src, void *dst, void *sink,
                                                      uint64_t steps, int32_t r, int32_t w,
                                                      int32_t blocks, void *stream) {
  if (blocks < 1) return (int)hipErrorInvalidValue;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (r == 1 && w == 0) return (int)launch_stream<1, 0>(src, dst, sink, steps, blocks, st);
  if (r == 0 && w == 1) return (int)launch_stream<0, 1>(src, dst, sink, steps, blocks, st);
  if (r == 1 && w == 1) return (int)launch_stream<1, 1>(src, dst, sink, steps, blocks, st);
  if (r == 2 && w == 1) return (int)launch_stream<2, 1>(src, dst, sink, steps, blocks, st);
  if (r == 4 && w == 1) return (int)launch_stream<4, 1>(src, dst, sink, steps, blocks, st);
  return (int)hipErrorInvalidValue;
}

__attribute__((visibility("default"))) int kvc_scatter_rows(
    const void *src, int64_t src_pitch, int32_t src_row_bytes, const int32_t *slots,
    int32_t n_rows, void *dst, int32_t row_bytes, int32_t block_size, int64_t dst_pitch,
    int64_t block_stride, int32_t num_slots, int32_t blocks, void *stream) {
  if (blocks < 1 || n_rows < 0 || block_size < 1 || src_row_bytes % 16 != 0 ||
      row_bytes % 16 != 0 || src_row_bytes > 2048 || row_bytes > 2048 ||
      src_pitch % 16 != 0 || dst_pitch % 16 != 0 || block_stride % 16 != 0)
    return (int)hipErrorInvalidValue;
  if (n_rows == 0) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint8_t *s = static_cast<const uint8_t *>(src);
  uint8_t *d = static_cast<uint8_t *>(dst);
  if (src_row_bytes <= 256 && row_bytes <= 256)  // 16 lanes a row, one piece each
    hipLaunchKernelGGL((scatter_kernel<16, 1>), dim3(blocks), dim3(256), 0, st, s, src_pitch,
                       src_row_bytes, slots, n_rows, d, row_bytes, block_size, dst_pitch,
                       block_stride, num_slots);
  else  // 32 lanes a row, up to four pieces each (rows up to 2 KiB)
    hipLaunchKernelGGL((scatter_kernel<32, 4>), dim3(blocks), dim3(256), 0, st, s, src_pitch,
                       src_row_bytes, slots, n_rows, d, row_bytes, block_size, dst_pitch,
                       block_stride, num_slots);
  return (int)hipGetLastError();
}

__attribute__((visibility("default"))) int kvc_clock(unsigned long long *out, int32_t spins,
                                                     void *stream) {
  if (out == nullptr || spins < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(clock_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), out,
                     spins);
  return (int)hipGetLastError();
}

__attribute__((visibility("default"))) int kvc_empty(int32_t blocks, void *stream) {
  if (blocks < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream));
  return (int)hipGetLastError();
}

}  // extern "C"
