// Roofline probes for the fused decode: the achievable HBM streaming-read rate and
// the LDS random-lookup rate of the decode tables, measured on the device the
// library runs on (the ceilings the decode kernel is compared against).
#include <hip/hip_runtime.h>

#include <string>

#include "ecw_internal.h"

namespace ecw {

// Streaming read: every thread reads 16-byte vectors in a grid-stride loop, four
// loads in flight, and folds them into one word so the loads cannot be dropped.
__global__ void __launch_bounds__(256) k_stream_read(const uint4* __restrict__ p, uint64_t n16, uint32_t* out) {
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  out[(uint64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// Per-wave tile streams, shaped like the decode's reads of its word and raw-byte
// planes: wave w reads its own contiguous region of `kib` KiB as 1 KiB wave-wide
// loads (16 bytes per lane), INFL of them in flight, with the decode's XCD-contiguous
// block order, and folds them into one word per lane so the loads cannot be dropped.
template <int INFL>
__global__ void __launch_bounds__(1024) k_tile_stream(const uint4* __restrict__ p, uint32_t kib, uint32_t n_waves,
                                                      uint32_t grid, uint32_t* out) {
  const uint32_t per = grid >> 3;
  const uint32_t gl = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  const uint32_t w = gl * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (w >= n_waves) return;
  const uint32_t lane = threadIdx.x & 63;
  const uint4* q = p + (uint64_t)w * kib * 64 + lane;
  uint32_t acc = 0;
  for (uint32_t k = 0; k < kib; k += INFL) {
    uint4 v[INFL];
#pragma unroll
    for (int i = 0; i < INFL; ++i) v[i] = k + i < kib ? q[(uint64_t)(k + i) * 64] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < INFL; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  out[(uint64_t)w * 64 + lane] = acc;
}

// LDS random lookups shaped like the decode: a table of 2^m entries of 4, 8, 12 or 16 bytes,
// and per lane a dependent chain idx -> entry -> next idx (the state update of the
// decode is a multiply-add on the entry).  Every wave of the chip runs `steps` steps.
template <int EB>
__global__ void __launch_bounds__(1024) k_lds_lookup(uint32_t log2m, uint32_t steps, uint32_t* out) {
  extern __shared__ __align__(16) unsigned char smem[];
  const uint32_t n = 1u << log2m, mask = n - 1u;
  for (uint32_t i = threadIdx.x; i < n * (EB / 4); i += blockDim.x)
    reinterpret_cast<uint32_t*>(smem)[i] = i * 2654435761u;
  __syncthreads();
  uint32_t x = (blockIdx.x * blockDim.x + threadIdx.x) * 2246822519u + 1u;
  for (uint32_t s = 0; s < steps; ++s) {
    const uint32_t slot = x & mask;
    if constexpr (EB == 12) {
      typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
      const u32x3 e = *reinterpret_cast<const u32x3*>(smem + slot * 12);
      x = __umul24(x >> log2m, e.x | 1u) + ((e.y ^ e.z) >> 16) + 0x9E37u;
    } else if constexpr (EB == 16) {
      const uint4 e = reinterpret_cast<const uint4*>(smem)[slot];
      x = __umul24(x >> log2m, e.x | 1u) + ((e.y ^ e.z ^ e.w) >> 16) + 0x9E37u;
    } else if constexpr (EB == 8) {
      const uint2 e = reinterpret_cast<const uint2*>(smem)[slot];
      x = __umul24(x >> log2m, e.x | 1u) + (e.y >> 16) + 0x9E37u;
    } else {
      const uint32_t e = reinterpret_cast<const uint32_t*>(smem)[slot];
      x = __umul24(x >> log2m, e | 1u) + (e >> 20) + 0x9E37u;
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = x;
}

// Shader clock under load: each one-wave block keeps a short dependent FMA chain
// busy until `ticks` of the constant-rate real-time counter have passed, and records
// how far the shader-clock counter moved meanwhile (lane 0: [cycles, ticks]).  Run
// beside another kernel, it reads the clock that kernel runs at.  The loop ends on
// the real-time bound or, should that counter not advance, after max_iters.
__global__ void __launch_bounds__(64) k_clock(uint64_t ticks, uint64_t max_iters, uint64_t* out) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  float a = (float)threadIdx.x;
  uint64_t r = r0;
  for (uint64_t it = 0; it < max_iters && r - r0 < ticks; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) a = fmaf(a, 0.999f, 0.25f);
    r = __builtin_amdgcn_s_memrealtime();
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = c1 - c0;
    out[2 * blockIdx.x + 1] = (r - r0) + (a == 12345.0f ? 1u : 0u);
  }
}

static ecw_status launch_error(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ECW_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return ECW_OK;
}

}  // namespace ecw

using namespace ecw;

extern "C" ecw_status ecw_probe_stream_read(ecw_stream stream, const void* buf, size_t bytes, uint32_t* sink,
                                            uint32_t blocks) {
  clear_error();
  if (!buf || !sink || blocks == 0 || bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16)
    return fail(ECW_E_INVALID_ARG, "stream probe: bad buffer, sink or block count");
  hipLaunchKernelGGL(k_stream_read, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const uint4*>(buf), (uint64_t)(bytes / 16), sink);
  return launch_error("stream probe launch failed");
}

extern "C" ecw_status ecw_probe_tile_stream(ecw_stream stream, const void* buf, size_t bytes, uint32_t kib_per_wave,
                                            uint32_t waves, uint32_t waves_per_block, uint32_t inflight,
                                            uint32_t* sink) {
  clear_error();
  if (!buf || !sink || reinterpret_cast<uintptr_t>(buf) % 16 || kib_per_wave == 0 || waves == 0 ||
      waves_per_block == 0 || waves_per_block > 16 || (inflight != 1 && inflight != 2 && inflight != 4) ||
      (uint64_t)waves * kib_per_wave * 1024u > bytes)
    return fail(ECW_E_INVALID_ARG, "tile stream probe: bad buffer, sink or shape");
  const uint32_t blocks = (waves + waves_per_block - 1) / waves_per_block;
  const uint32_t grid = (blocks + 7) / 8 * 8;
  auto fn = inflight == 4 ? k_tile_stream<4> : inflight == 2 ? k_tile_stream<2> : k_tile_stream<1>;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(waves_per_block * 64), 0, (hipStream_t)stream,
                     static_cast<const uint4*>(buf), kib_per_wave, waves, grid, sink);
  return launch_error("tile stream probe launch failed");
}

extern "C" ecw_status ecw_probe_lds_lookup(ecw_stream stream, uint32_t log2_m, uint32_t entry_bytes,
                                           uint32_t steps, uint32_t blocks, uint32_t waves_per_block,
                                           uint32_t* sink) {
  clear_error();
  if (!sink || log2_m < 8 || log2_m > 13 ||
      (entry_bytes != 4 && entry_bytes != 8 && entry_bytes != 12 && entry_bytes != 16) ||
      (entry_bytes << log2_m) > 160u * 1024u || blocks == 0 ||
      waves_per_block == 0 || waves_per_block > 16)
    return fail(ECW_E_INVALID_ARG, "lookup probe: bad arguments");
  const size_t lds = ((size_t)entry_bytes) << log2_m;
  auto fn = entry_bytes == 16 ? k_lds_lookup<16>
             : entry_bytes == 12 ? k_lds_lookup<12>
             : entry_bytes == 8 ? k_lds_lookup<8> : k_lds_lookup<4>;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                          160 * 1024) != hipSuccess) {
    (void)hipGetLastError();
    return fail(ECW_E_HIP, "hipFuncSetAttribute failed");
  }
  hipLaunchKernelGGL(fn, dim3(blocks), dim3(waves_per_block * 64), lds, (hipStream_t)stream, log2_m, steps, sink);
  return launch_error("lookup probe launch failed");
}

extern "C" ecw_status ecw_probe_clock(ecw_stream stream, uint32_t duration_us, uint32_t blocks, uint64_t* sink,
                                      uint32_t* wall_clock_khz) {
  clear_error();
  if (!sink || !wall_clock_khz || blocks == 0 || duration_us == 0 || duration_us > 1000000)
    return fail(ECW_E_INVALID_ARG, "clock probe: bad arguments");
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
      khz <= 0) {
    (void)hipGetLastError();
    return fail(ECW_E_HIP, "wall clock rate unavailable");
  }
  *wall_clock_khz = (uint32_t)khz;
  const uint64_t ticks = (uint64_t)khz * duration_us / 1000u;
  hipLaunchKernelGGL(k_clock, dim3(blocks), dim3(64), 0, (hipStream_t)stream, ticks, (uint64_t)duration_us * 1000u,
                     sink);
  return launch_error("clock probe launch failed");
}
