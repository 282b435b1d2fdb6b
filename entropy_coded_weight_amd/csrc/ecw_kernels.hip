// Fused rANS decode + batch-1..4 GEMV for gfx950, and the decode-only test hook.
//
// One wave64 decodes one tile at a time: lane l owns row 64g + l (MINE page,
// Section 4 "Grid Layout": one lane per row, tiles stacked into blocks that share
// the activation slice), tiles are independent rANS streams with 32-bit states and
// 16-bit words (EntroPack page, Sections 3.6 and C.3).  Per step and lane:
//
//   slot = x & (M-1);  e = LUT[slot]            (LDS, one 8-byte read)
//   x    = f * (x >> m) + bias                  (v_mad_u32_u24)
//   weight from e's payload byte                (+ raw byte for BF16)
//   acc += weight * x_col                        (fp32)
//   need = x < 2^16; off = popcount(ballot(need) below this lane)
//   if need: x = x << 16 | word[pos + off];  pos += popcount(ballot)
//
// The words of a wave's run of tiles are contiguous in HBM; they are streamed into
// a per-wave LDS ring in 1 KiB chunks (64 lanes x 16 B, one coalesced load per
// lane), one chunk prefetched in registers ahead of use.  The table is staged in
// LDS once per block (MINE page, Section 4.1: decoding tables in shared memory,
// 1 KiB per-warp chunk buffer for the stream).  No weight tensor is written:
// weights live in registers between decode and FMA.
//
// Cross-wave reduction: the waves of a block cover consecutive column slices of
// the same 64 rows and are summed in LDS in wave order; when a row group spans
// several blocks each block writes a partial and a second small kernel sums them in
// block order.  Both orders are fixed, so results do not depend on scheduling.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <unordered_set>

#include "ecw_internal.h"

namespace ecw {

constexpr uint32_t kRing = 1024;          // words per wave ring (two chunks)
constexpr uint32_t kMirror = 64;          // copy of the ring head for reads that wrap
constexpr uint32_t kRingStride = kRing + kMirror;
constexpr uint32_t kChunk = 512;          // words per chunk = 64 lanes x 16 bytes

constexpr int kMaxGroup = 8;

// Per-tensor launch arguments (one entry per tensor of a grouped launch).
struct TArgs {
  const uint2* lut;
  const uint32_t* states;
  const uint32_t* offsets;
  const uint16_t* words;
  const uint8_t* raw;
  const uint16_t* scales;
  const void* x;
  float* y;
  float* partials;
  uint16_t* sym_out;
  void* w_out;
  uint32_t* status_out;
  uint32_t rows, cols, n_rg, n_sl, s_full, s_last, log2m, tile_cols;
  uint32_t tiles_per_wave, n_sg, n_blocks, block_begin, syms_per_row;
  uint32_t x_is_bf16, nb, lut_entries, xs_cols;
  uint32_t raw_full_bytes, raw_rg_bytes;
};

struct KArgs {
  TArgs t[kMaxGroup];
  uint32_t nt;           // tensors in the launch
  uint32_t n_blocks;     // total logical blocks
};

__device__ __forceinline__ float load_x(const void* x, uint32_t is_bf16, uint64_t i) {
  const uint16_t h = static_cast<const uint16_t*>(x)[i];
  if (is_bf16) return __uint_as_float((uint32_t)h << 16);
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ float wave_sum(float v) {
  // fixed xor-butterfly: every lane ends with the same, order-independent-of-timing sum
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// x' = f * (x >> m) + bias in one v_mad_u32_u24 (both factors < 2^24; the payload
// byte in bits 24..31 of the table word is ignored by the 24-bit multiply).
__device__ __forceinline__ uint32_t mad_u24(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t d;
  asm("v_mad_u32_u24 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// acc + f16(h >> 16) * x in fp32 (v_fma_mix_f32: operand 0 is the fp16 in the high
// half of h, operands 1 and 2 are fp32).  Exact widening of the fp16 weight.
__device__ __forceinline__ float fma_mix_hi(uint32_t h, float x, float acc) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "=v"(d) : "v"(h), "v"(x), "v"(acc));
  return d;
}

// Per lane: mask bit set ? t : f (v_cndmask on a wave-uniform lane mask).  Inline
// asm so the compiler cannot turn it back into an exec-masked branch.
__device__ __forceinline__ uint32_t select_lanes(uint64_t mask, uint32_t t, uint32_t f) {
  uint32_t d;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(d) : "v"(f), "v"(t), "s"(mask));
  return d;
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// ---- the per-stream pieces of one decode step (scalar state, kept in registers)

// A4: one symbol decode.  Returns the table entry (f | a8 << 24, bias | h16 << 16).
__device__ __forceinline__ uint2 decode_step(uint32_t& x, const uint2* lut, uint32_t m, uint32_t mmask) {
  const uint2 e = lut[x & mmask];
  x = mad_u24(x >> m, e.x, e.y & 0xFFFFu);
  return e;
}

// A5: renormalise the wave's 64 states against the stream's LDS ring; refill the
// ring one chunk ahead of the read position (the chunk was loaded into `pre`
// one chunk-consumption earlier).
template <bool RAGGED>
__device__ __forceinline__ void renorm_step(uint32_t& x, uint32_t& rpos, uint32_t& have, uint32_t& nc,
                                            uint4& pre, uint16_t* ring, const uint4* src, uint32_t nch,
                                            uint32_t lane, bool active) {
  if (rpos + 64 > have) {            // wave-uniform
    const uint32_t slot_c = nc & 1u;
    reinterpret_cast<uint4*>(ring + slot_c * kChunk)[lane] = pre;
    if (slot_c == 0 && lane < 8) reinterpret_cast<uint4*>(ring + kRing)[lane] = pre;
    have += kChunk;
    ++nc;
    if (nc < nch) pre = src[(uint64_t)nc * 64];
  }
  // Branch-free: every lane reads the word at its prefix offset (always inside the
  // ring plus its mirror) and keeps it only if it needs one, so no exec-mask
  // change or LDS wait splits the step.
  const uint16_t* rp = ring + (rpos & (kRing - 1));
  uint64_t msk;
  if constexpr (RAGGED)
    msk = __ballot(active && (x < kStateL));
  else
    msk = __builtin_amdgcn_ballot_w64(x < kStateL);
  const uint32_t w = rp[lanes_below(msk)];
  x = select_lanes(msk, (x << 16) | w, x);
  rpos += (uint32_t)__popcll(msk);
}

// A6 + A7: rebuild the weight(s) of one symbol in registers and accumulate.
// xp: this symbol's activations, [KW][B] floats.  r: BF16 raw byte.
template <int PAY, int CB, int KW, int B>
__device__ __forceinline__ void mac(const uint2 e, const float* xp, uint32_t r, float* acc) {
  if constexpr (PAY == 1) {
    if constexpr (KW == 1) {
#pragma unroll
      for (int b = 0; b < B; ++b) acc[b] = fma_mix_hi(e.y, xp[b], acc[b]);        // q0
    } else if constexpr (KW == 2) {
      const float w0 = (float)(int8_t)(e.x >> 24);                                // q0
#pragma unroll
      for (int b = 0; b < B; ++b) {
        acc[b] = fmaf(w0, xp[b], acc[b]);
        acc[b] = fma_mix_hi(e.y, xp[B + b], acc[b]);                             // q1
      }
    } else {
#pragma unroll
      for (int i = 0; i < KW; ++i) {
        const float w = (float)((int)((e.x >> (24 + CB * i)) & ((1u << CB) - 1)) - (1 << (CB - 1)));
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = fmaf(w, xp[i * B + b], acc[b]);
      }
    }
  } else if constexpr (PAY == 2) {
    // bf16 bits = sign << 15 | exponent << 7 | mantissa, as fp32 bits << 16
    const uint32_t bits = ((r << 24) & 0x80000000u) | ((e.x >> 1) & 0x7F800000u) | ((r << 16) & 0x007F0000u);
    const float w = __uint_as_float(bits);
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = fmaf(w, xp[b], acc[b]);
  } else {
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = fma_mix_hi(e.y, xp[b], acc[b]);          // e4m3 value
  }
}

__device__ __forceinline__ uint32_t raw_byte(const uint4& g, int u) {
  const uint32_t dw = (u < 4) ? g.x : (u < 8) ? g.y : (u < 12) ? g.z : g.w;
  return (dw >> (8 * (u & 3))) & 0xFFu;
}

__device__ __forceinline__ const uint8_t* raw_tile(const TArgs& a, uint32_t rg, uint32_t sl, uint32_t lane) {
  return a.raw + (uint64_t)rg * a.raw_rg_bytes + (uint64_t)sl * a.raw_full_bytes + lane * 16;
}

// Word range of a run of tiles [t0, t1): chunk-aligned start, chunk count, first
// read position.
__device__ __forceinline__ void run_words(const TArgs& a, uint32_t t0, uint32_t t1, uint32_t& gb,
                                          uint32_t& nch, uint32_t& rpos) {
  if (t0 >= t1) {
    gb = 0; nch = 0; rpos = 0;
    return;
  }
  const uint32_t wb = a.offsets[t0], we = a.offsets[t1];
  gb = wb & ~(kChunk - 1);
  nch = (we - gb + kChunk - 1) / kChunk;
  rpos = wb - gb;
}

// The wave body.  NS = 1: the wave's tiles [t0, t1) are one stream.  NS = 2: the
// first half (stream A) and the second half (stream B) are decoded in lockstep, two
// independent dependency chains per wave.  MAT: decode-only test hook (NS = 1).
// The first two chunks of each stream (c0*, c1*) were loaded by the caller before
// the block's staging barrier and are committed to the rings here.
template <int PAY, int CB, int KW, int B, bool MAT, bool RAGGED, int NS>
__device__ __forceinline__ void wave_body(const TArgs& a, const uint2* lut, const float* xs, uint16_t* ring,
                                          uint32_t rg, uint32_t tA0, uint32_t tA1, uint32_t tB0,
                                          uint32_t tB1, uint32_t c_lo, uint32_t lane, bool active,
                                          float* acc) {
  constexpr int U = 16;
  const uint32_t m = a.log2m, mmask = (1u << m) - 1u;
  const uint32_t row = rg * 64 + lane;
  const uint32_t sl0 = rg * a.n_sl;
  const uint4 zero4 = {0u, 0u, 0u, 0u};
  uint16_t* ringA = ring;
  uint16_t* ringB = ring + kRingStride;

  uint32_t gbA, nchA, rposA, gbB = 0, nchB = 0, rposB = 0;
  run_words(a, tA0, tA1, gbA, nchA, rposA);
  if constexpr (NS == 2) run_words(a, tB0, tB1, gbB, nchB, rposB);
  const uint4* srcA = reinterpret_cast<const uint4*>(a.words + gbA) + lane;
  const uint4* srcB = reinterpret_cast<const uint4*>(a.words + gbB) + lane;
  // first chunks (issued together; they travel while the previous stream's
  // staging finishes) and the one-ahead prefetch
  {
    const uint4 c0 = nchA > 0 ? srcA[0] : zero4;
    const uint4 c1 = nchA > 1 ? srcA[64] : zero4;
    uint4 d0 = zero4, d1 = zero4;
    if constexpr (NS == 2) {
      d0 = nchB > 0 ? srcB[0] : zero4;
      d1 = nchB > 1 ? srcB[64] : zero4;
    }
    reinterpret_cast<uint4*>(ringA)[lane] = c0;
    if (lane < 8) reinterpret_cast<uint4*>(ringA + kRing)[lane] = c0;
    reinterpret_cast<uint4*>(ringA + kChunk)[lane] = c1;
    if constexpr (NS == 2) {
      reinterpret_cast<uint4*>(ringB)[lane] = d0;
      if (lane < 8) reinterpret_cast<uint4*>(ringB + kRing)[lane] = d0;
      reinterpret_cast<uint4*>(ringB + kChunk)[lane] = d1;
    }
  }
  uint4 preA = nchA > 2 ? srcA[128] : zero4;
  uint4 preB = zero4;
  if constexpr (NS == 2) preB = nchB > 2 ? srcB[128] : zero4;
  uint32_t haveA = 2 * kChunk, ncA = 2, haveB = 2 * kChunk, ncB = 2;
  uint32_t stA = tA0 < tA1 ? a.states[(uint64_t)tA0 * 64 + lane] : kStateL;
  uint32_t stB = kStateL;
  if constexpr (NS == 2) stB = tB0 < tB1 ? a.states[(uint64_t)tB0 * 64 + lane] : kStateL;

  uint32_t tA = tA0, tB = tB0;
  while (tA < tA1) {
    const bool pairB = (NS == 2) && (tB < tB1);           // wave-uniform
    uint32_t xA = stA, xB = stB;
    if (tA + 1 < tA1) stA = a.states[(uint64_t)(tA + 1) * 64 + lane];
    if constexpr (NS == 2) {
      if (pairB && tB + 1 < tB1) stB = a.states[(uint64_t)(tB + 1) * 64 + lane];
    }
    const uint32_t slA = tA - sl0, slB = tB - sl0;
    const uint32_t SA = (slA + 1 == a.n_sl) ? a.s_last : a.s_full;
    const uint32_t SB = pairB ? ((slB + 1 == a.n_sl) ? a.s_last : a.s_full) : 0;   // SB <= SA
    const uint32_t colA = slA * a.tile_cols - c_lo, colB = slB * a.tile_cols - c_lo;
    const uint8_t* rawA = raw_tile(a, rg, slA, lane);
    const uint8_t* rawB = raw_tile(a, rg, slB, lane);

    for (uint32_t j = 0; j < SA; j += U) {
      const bool dualB = j < SB;                            // wave-uniform
      uint4 rgA = zero4, rgB = zero4;
      if constexpr (PAY == 2) {
        rgA = *reinterpret_cast<const uint4*>(rawA + (uint64_t)(j / U) * 1024);
        if (NS == 2 && dualB) rgB = *reinterpret_cast<const uint4*>(rawB + (uint64_t)(j / U) * 1024);
      }
      const float4* xgA = reinterpret_cast<const float4*>(xs + (uint64_t)(colA + KW * j) * B);
      const float4* xgB = reinterpret_cast<const float4*>(xs + (uint64_t)(colB + KW * j) * B);
#pragma unroll
      for (int qtr = 0; qtr < U / 4; ++qtr) {
        float4 xqA[MAT ? 1 : KW * B], xqB[MAT ? 1 : KW * B];
        if constexpr (!MAT) {
#pragma unroll
          for (int i = 0; i < KW * B; ++i) xqA[i] = xgA[qtr * KW * B + i];
          if (NS == 2 && dualB) {
#pragma unroll
            for (int i = 0; i < KW * B; ++i) xqB[i] = xgB[qtr * KW * B + i];
          }
        }
#pragma unroll
        for (int u4 = 0; u4 < 4; ++u4) {
          const int u = qtr * 4 + u4;
          const uint32_t step = j + u;
          const uint2 eA = decode_step(xA, lut, m, mmask);
          uint2 eB = {0u, 0u};
          if (NS == 2 && dualB) eB = decode_step(xB, lut, m, mmask);
          if constexpr (!MAT) {
            mac<PAY, CB, KW, B>(eA, reinterpret_cast<const float*>(xqA) + u4 * KW * B,
                                PAY == 2 ? raw_byte(rgA, u) : 0u, acc);
            if (NS == 2 && dualB)
              mac<PAY, CB, KW, B>(eB, reinterpret_cast<const float*>(xqB) + u4 * KW * B,
                                  PAY == 2 ? raw_byte(rgB, u) : 0u, acc);
          } else if (!RAGGED || active) {
            const uint32_t aux = eA.x >> 24;
            uint32_t symbol = aux;
            int q[KW > 0 ? KW : 1];
            if constexpr (PAY == 1) {
              constexpr int half = 1 << (CB - 1);
              if constexpr (KW == 4) {
#pragma unroll
                for (int i = 0; i < KW; ++i) q[i] = (int)((aux >> (CB * i)) & ((1u << CB) - 1)) - half;
              } else {
                q[0] = (int)(int8_t)aux;
                if constexpr (KW == 2) q[1] = (int)(float)__builtin_bit_cast(_Float16, (uint16_t)(eA.y >> 16));
                symbol = 0;
#pragma unroll
                for (int i = 0; i < KW; ++i) symbol |= (uint32_t)(q[i] + half) << (CB * i);
              }
            }
            if (a.sym_out) a.sym_out[(uint64_t)row * a.syms_per_row + (uint64_t)slA * a.s_full + step] = (uint16_t)symbol;
            if (a.w_out) {
              const uint64_t wi = (uint64_t)row * a.cols + (uint64_t)slA * a.tile_cols + (uint64_t)step * KW;
              if constexpr (PAY == 1) {
#pragma unroll
                for (int i = 0; i < KW; ++i) static_cast<int8_t*>(a.w_out)[wi + i] = (int8_t)q[i];
              } else if constexpr (PAY == 2) {
                const uint32_t r = raw_byte(rgA, u);
                static_cast<uint16_t*>(a.w_out)[wi] = (uint16_t)(((r & 0x80u) << 8) | (aux << 7) | (r & 0x7Fu));
              } else {
                static_cast<uint8_t*>(a.w_out)[wi] = (uint8_t)aux;
              }
            }
          }
          renorm_step<RAGGED>(xA, rposA, haveA, ncA, preA, ringA, srcA, nchA, lane, active);
          if (NS == 2 && dualB) renorm_step<RAGGED>(xB, rposB, haveB, ncB, preB, ringB, srcB, nchB, lane, active);
        }
      }
    }
    if constexpr (MAT) {
      const bool ok_lane = !active || xA == kStateL;
      const uint64_t bad = __ballot(!ok_lane);
      if (lane == 0 && a.status_out)
        a.status_out[tA] = (bad != 0 ? 1u : 0u) | ((rposA != a.offsets[tA + 1] - gbA) ? 2u : 0u);
    }
    ++tA;
    if (pairB) ++tB;
  }
}

// PAY: 1 INT codes, 2 BF16 exponent, 3 FP8.  CB/KW: code bits and codes per symbol
// (INT).  B: batch capacity (1 or 4).  MAT: decode-only test hook.
// Block = W waves on consecutive slices of one row group; wave w owns R tiles,
// decoded as one stream or, when R >= 2 and the payload allows, two interleaved
// streams (the host sizes the LDS rings the same way).
template <int PAY, int CB, int KW, int B, bool MAT>
__global__ void __launch_bounds__(1024) k_decode(const KArgs ka) {
  extern __shared__ __align__(16) unsigned char smem[];
  const uint32_t W = blockDim.x >> 6;
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wid = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Hardware block b runs on XCD b % 8.  Give each XCD a contiguous range of logical
  // blocks (the slice groups of one row group are adjacent).  gridDim.x is a
  // multiple of 8; surplus blocks exit at once.
  const uint32_t per = gridDim.x >> 3;
  const uint32_t gl = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (gl >= ka.n_blocks) return;
  // tensor of a grouped launch: blocks are numbered tensor by tensor
  uint32_t ti = 0;
  for (uint32_t i = 1; i < ka.nt; ++i)
    if (gl >= ka.t[i].block_begin) ti = i;
  const TArgs& a = ka.t[ti];
  const uint32_t lb = gl - a.block_begin;
  const uint32_t rg = lb / a.n_sg, sg = lb - rg * a.n_sg;
  const uint32_t R = a.tiles_per_wave;
  const uint32_t sl_blk = sg * W * R;
  const uint32_t sl_blk_end = min(sl_blk + W * R, a.n_sl);
  const uint32_t c_lo = sl_blk * a.tile_cols;
  const uint32_t c_hi = min(sl_blk_end * a.tile_cols, a.cols);
  constexpr bool kTwoCapable = !MAT && PAY != 2 && KW != 4;
  const uint32_t NSr = (kTwoCapable && R >= 2) ? 2 : 1;

  const uint32_t lut_bytes = a.lut_entries * 8;
  uint2* lut = reinterpret_cast<uint2*>(smem);
  float* xs = reinterpret_cast<float*>(smem + lut_bytes);
  const uint32_t xs_bytes = MAT ? 0 : ((a.xs_cols * B * 4 + 15) & ~15u);
  uint16_t* rings = reinterpret_cast<uint16_t*>(smem + lut_bytes + xs_bytes);
  uint16_t* ring = rings + (wid * NSr) * kRingStride;

  // ---- A2: stage the decode table (two 16-byte loads in flight per thread)
  {
    const uint4* src = reinterpret_cast<const uint4*>(a.lut);
    uint4* dst = reinterpret_cast<uint4*>(lut);
    const uint32_t n = a.lut_entries / 2, bd = blockDim.x;
    for (uint32_t i = tid; i < n; i += 2 * bd) {
      const uint32_t i2 = i + bd;
      const uint4 v0 = src[i];
      const uint4 v1 = src[i2 < n ? i2 : i];
      dst[i] = v0;
      if (i2 < n) dst[i2] = v1;
    }
  }
  // ---- A3: stage the block's activation columns as fp32 [col][b], 8 columns
  // (16 bytes) per load
  if constexpr (!MAT) {
    const uint32_t nvec = a.xs_cols / 8;
    for (uint32_t v = tid; v < nvec * B; v += blockDim.x) {
      const uint32_t b = v / nvec, c8 = v - b * nvec, col = c_lo + 8 * c8;
      uint4 raw = {0u, 0u, 0u, 0u};
      if (col < c_hi && b < a.nb)
        raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + (uint64_t)b * a.cols + col);
      const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint16_t h = (uint16_t)(w4[i >> 1] >> (16 * (i & 1)));
        xs[(8 * c8 + i) * B + b] = a.x_is_bf16 ? __uint_as_float((uint32_t)h << 16)
                                               : (float)__builtin_bit_cast(_Float16, h);
      }
    }
  }
  __syncthreads();

  const uint32_t w_sl0 = min(sl_blk + wid * R, sl_blk_end);
  const uint32_t w_sl1 = min(w_sl0 + R, sl_blk_end);
  const uint32_t w_mid = NSr == 1 ? w_sl1 : w_sl0 + (w_sl1 - w_sl0 + 1) / 2;
  const uint32_t tb = rg * a.n_sl;
  const uint32_t row = rg * 64 + lane;
  const bool active = row < a.rows;
  const bool ragged = (rg + 1) * 64 > a.rows;     // wave-uniform
  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.f;
  if (w_sl0 < w_sl1) {
    if constexpr (kTwoCapable) {
      if (NSr == 2) {
        if (ragged)
          wave_body<PAY, CB, KW, B, MAT, true, 2>(a, lut, xs, ring, rg, tb + w_sl0, tb + w_mid, tb + w_mid,
                                                  tb + w_sl1, c_lo, lane, active, acc);
        else
          wave_body<PAY, CB, KW, B, MAT, false, 2>(a, lut, xs, ring, rg, tb + w_sl0, tb + w_mid, tb + w_mid,
                                                   tb + w_sl1, c_lo, lane, active, acc);
      }
    }
    if (NSr == 1) {
      if (ragged)
        wave_body<PAY, CB, KW, B, MAT, true, 1>(a, lut, xs, ring, rg, tb + w_sl0, tb + w_sl1, 0, 0, c_lo,
                                                lane, active, acc);
      else
        wave_body<PAY, CB, KW, B, MAT, false, 1>(a, lut, xs, ring, rg, tb + w_sl0, tb + w_sl1, 0, 0, c_lo,
                                                 lane, active, acc);
    }
  }
  if constexpr (!MAT) {
    // ---- A8: epilogue.  Reuse this wave's first ring as its reduction slot.
    float* red = reinterpret_cast<float*>(ring);
#pragma unroll
    for (int b = 0; b < B; ++b) red[b * 64 + lane] = acc[b];
    __syncthreads();
    for (uint32_t i = tid; i < 64u * B; i += blockDim.x) {
      const uint32_t b = i >> 6, l = i & 63, r = rg * 64 + l;
      float s = 0.f;
      for (uint32_t w = 0; w < W; ++w)
        s += reinterpret_cast<const float*>(rings + (w * NSr) * kRingStride)[b * 64 + l];
      if (a.n_sg == 1) {
        if (r < a.rows && b < a.nb) {
          const float sc = (PAY == 2) ? 1.f : (float)__builtin_bit_cast(_Float16, a.scales[r]);
          a.y[(uint64_t)b * a.rows + r] = s * sc;
        }
      } else {
        a.partials[(((uint64_t)rg * a.n_sg + sg) * B + b) * 64 + l] = s;
      }
    }
  }
}

// Fixed-order sum of the per-block partials of each row (row groups that span
// several blocks), times the row scale.  A separate launch: the kernel boundary
// makes the partials visible without device-wide cache flushes.  One launch covers
// every tensor of a group that needs it.
struct RArgs {
  const float* partials[kMaxGroup];
  const uint16_t* scales[kMaxGroup];
  float* y[kMaxGroup];
  uint32_t rows[kMaxGroup], n_sg[kMaxGroup], row_begin[kMaxGroup];
  uint32_t nt, nb, unit_scale, total_rows;
};

template <int B>
__global__ void __launch_bounds__(256) k_reduce(const RArgs ra) {
  const uint32_t gi = blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= ra.total_rows) return;
  uint32_t ti = 0;
  for (uint32_t i = 1; i < ra.nt; ++i)
    if (gi >= ra.row_begin[i]) ti = i;
  const uint32_t r = gi - ra.row_begin[ti], rg = r >> 6, l = r & 63, n_sg = ra.n_sg[ti];
  const float sc = ra.unit_scale ? 1.f : (float)__builtin_bit_cast(_Float16, ra.scales[ti][r]);
#pragma unroll
  for (int b = 0; b < B; ++b) {
    if ((uint32_t)b >= ra.nb) break;
    float s = 0.f;
    for (uint32_t g = 0; g < n_sg; ++g) s += ra.partials[ti][(((uint64_t)rg * n_sg + g) * B + b) * 64 + l];
    ra.y[ti][(uint64_t)b * ra.rows[ti] + r] = s * sc;
  }
}

__global__ void k_fill_zero(float* y, uint64_t n) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = 0.f;
}

// ------------------------------------------------------------------ host launch
using KernelFn = void (*)(const KArgs);

template <int B, bool MAT>
static KernelFn pick_kernel(const ecw_coding& c) {
  switch (c.payload) {
    case ECW_P_INT_CODES:
      switch (c.code_bits * 16 + c.weights_per_symbol) {
        case 4 * 16 + 1: return k_decode<1, 4, 1, B, MAT>;
        case 4 * 16 + 2: return k_decode<1, 4, 2, B, MAT>;
        case 3 * 16 + 1: return k_decode<1, 3, 1, B, MAT>;
        case 3 * 16 + 2: return k_decode<1, 3, 2, B, MAT>;
        case 2 * 16 + 1: return k_decode<1, 2, 1, B, MAT>;
        case 2 * 16 + 2: return k_decode<1, 2, 2, B, MAT>;
        case 2 * 16 + 4: return k_decode<1, 2, 4, B, MAT>;
      }
      return nullptr;
    case ECW_P_BF16_EXP: return k_decode<2, 0, 1, B, MAT>;
    case ECW_P_FP8_E4M3: return k_decode<3, 0, 1, B, MAT>;
  }
  return nullptr;
}

static uint32_t streams_per_wave(const ecw_coding& c, bool mat, uint32_t R) {
  return (mat || c.payload == ECW_P_BF16_EXP || c.weights_per_symbol == 4 || R < 2) ? 1 : 2;
}

// Dynamic LDS of one block: decode table, staged activations, word rings.
static uint64_t lds_bytes(const ecw_tensor* t, uint32_t W, uint32_t R, uint32_t xs_cols, int B, bool mat) {
  const uint64_t lut = (uint64_t)t->n_tables << t->coding.log2_m;
  uint64_t xs = mat ? 0 : ((uint64_t)xs_cols * B * 4 + 15) / 16 * 16;
  return lut * 8 + xs + (uint64_t)W * streams_per_wave(t->coding, mat, R) * kRingStride * 2;
}

// Allow each kernel the whole 160 KiB LDS once (a host call, not a stream
// operation, so launches stay capturable).
static bool lds_attribute_set(KernelFn fn) {
  static std::mutex mu;
  static std::unordered_set<const void*> done;
  std::lock_guard<std::mutex> lock(mu);
  const void* key = reinterpret_cast<const void*>(fn);
  if (done.count(key)) return true;
  if (hipFuncSetAttribute(key, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  done.insert(key);
  return true;
}

static void fill_tensor(const ecw_tensor* t, TArgs& a) {
  const uint8_t* base = static_cast<const uint8_t*>(t->device_blob);
  a.lut = reinterpret_cast<const uint2*>(base + t->off_lut);
  a.states = reinterpret_cast<const uint32_t*>(base + t->off_states);
  a.offsets = reinterpret_cast<const uint32_t*>(base + t->off_offsets);
  a.words = reinterpret_cast<const uint16_t*>(base + t->off_words);
  a.raw = base + t->off_raw;
  a.scales = reinterpret_cast<const uint16_t*>(base + t->off_scales);
  a.rows = t->coding.rows;
  a.cols = t->coding.cols;
  a.n_rg = t->n_row_groups;
  a.n_sl = t->n_slices;
  a.s_full = t->steps_full;
  a.s_last = t->steps_last;
  a.log2m = t->coding.log2_m;
  a.tile_cols = t->coding.tile_cols;
  a.syms_per_row = symbols_per_row(t->coding.payload, t->coding.weights_per_symbol, t->coding.cols);
  a.lut_entries = t->n_tables << t->coding.log2_m;
  a.raw_full_bytes = (uint32_t)(raw_group_count(t->steps_full) * 1024);
  a.raw_rg_bytes = t->n_slices ? (uint32_t)((t->n_slices - 1) * raw_group_count(t->steps_full) * 1024 +
                                            raw_group_count(t->steps_last) * 1024) : 0;
}

static ecw_status check_tensor(const ecw_tensor* t) {
  if (!t) return fail(ECW_E_INVALID_ARG, "tensor is NULL");
  ecw_status st = check_coding(&t->coding);
  if (st != ECW_OK) return st;
  if (!t->device_blob) return fail(ECW_E_INVALID_ARG, "tensor has no device blob");
  if (reinterpret_cast<uintptr_t>(t->device_blob) % 256) return fail(ECW_E_INVALID_ARG, "device blob misaligned");
  if (t->coding.payload == ECW_P_E8_LATTICE) return fail(ECW_E_UNSUPPORTED, "E8 lattice decode kernel not built");
  if (t->waves_per_block < 1 || t->waves_per_block > 16 || t->tiles_per_wave < 1 || t->tiles_per_wave > 4096)
    return fail(ECW_E_INVALID_ARG, "launch shape out of range");
  if (t->steps_full % 16 || t->steps_last % 16) return fail(ECW_E_UNSUPPORTED, "steps per tile must be a multiple of 16");
  return ECW_OK;
}

static uint64_t align256(uint64_t v) { return (v + 255) / 256 * 256; }

// Workspace layout of a group: each tensor whose row groups span several blocks
// gets its partials, in tensor order, 256-byte aligned.
static uint64_t group_workspace(const ecw_tensor* const* ts, int n, int batch, uint64_t* off) {
  uint64_t pos = 0;
  for (int i = 0; i < n; ++i) {
    const uint64_t w = workspace_bytes(ts[i], batch);
    if (off) off[i] = pos;
    pos += align256(w);
  }
  return pos;
}

static ecw_status check_group(const ecw_tensor* const* ts, int n, int batch, int x_dtype, const void* x,
                              float* const* ys) {
  if (!ts || n < 1 || n > kMaxGroup) return fail(ECW_E_INVALID_ARG, "group must hold 1..8 tensors");
  if (batch < 1 || batch > 4) return fail(ECW_E_INVALID_ARG, "batch must be 1..4");
  if (x_dtype != ECW_DT_F16 && x_dtype != ECW_DT_BF16) return fail(ECW_E_INVALID_ARG, "x dtype must be F16 or BF16");
  if (!ys) return fail(ECW_E_INVALID_ARG, "y array is NULL");
  for (int i = 0; i < n; ++i) {
    ecw_status st = check_tensor(ts[i]);
    if (st != ECW_OK) return st;
    const ecw_coding& c = ts[i]->coding, &c0 = ts[0]->coding;
    if (c.payload != c0.payload || c.code_bits != c0.code_bits || c.weights_per_symbol != c0.weights_per_symbol ||
        c.cols != c0.cols || ts[i]->waves_per_block != ts[0]->waves_per_block)
      return fail(ECW_E_INVALID_ARG, "grouped tensors must share payload, code width, cols and waves per block");
    if (c.rows && (!ys[i] || reinterpret_cast<uintptr_t>(ys[i]) % 16))
      return fail(ECW_E_INVALID_ARG, "y must be a 16-byte aligned device pointer");
  }
  if (ts[0]->coding.cols && (!x || reinterpret_cast<uintptr_t>(x) % 16))
    return fail(ECW_E_INVALID_ARG, "x must be a 16-byte aligned device pointer");
  return ECW_OK;
}

// Fused decode + GEMV of a group of tensors that read the same x (one launch),
// then one launch that adds the cross-block partials where a row group spans
// several blocks.
static ecw_status launch_group(ecw_stream stream, const ecw_tensor* const* ts, int n, const void* x,
                               int x_dtype, float* const* ys, int batch, void* workspace, size_t ws_bytes) {
  ecw_status st = check_group(ts, n, batch, x_dtype, x, ys);
  if (st != ECW_OK) return st;
  uint64_t woff[kMaxGroup];
  const uint64_t need = group_workspace(ts, n, batch, woff);
  if (need && (!workspace || ws_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256))
    return fail(ECW_E_INVALID_ARG, "workspace missing, too small or not 256-byte aligned");
  const int B = batch > 1 ? 4 : 1;
  const uint32_t W = ts[0]->waves_per_block;
  KArgs ka{};
  RArgs ra{};
  uint64_t lds = 0;
  uint32_t blocks = 0, red_rows = 0;
  for (int i = 0; i < n; ++i) {
    const ecw_tensor* t = ts[i];
    if (t->coding.rows == 0) continue;
    if (t->n_tiles == 0) {   // K == 0: y = 0 (a fill kernel keeps the call graph-capturable)
      const uint64_t cnt = (uint64_t)batch * t->coding.rows;
      hipLaunchKernelGGL(k_fill_zero, dim3((uint32_t)((cnt + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                         ys[i], cnt);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return fail(ECW_E_HIP, "fill launch failed");
      continue;
    }
    TArgs& a = ka.t[ka.nt];
    fill_tensor(t, a);
    a.x = x;
    a.y = ys[i];
    a.x_is_bf16 = x_dtype == ECW_DT_BF16;
    a.nb = (uint32_t)batch;
    a.tiles_per_wave = t->tiles_per_wave;
    a.n_sg = slice_groups(t);
    a.n_blocks = a.n_rg * a.n_sg;
    a.block_begin = blocks;
    a.xs_cols = W * t->tiles_per_wave * t->coding.tile_cols;
    blocks += a.n_blocks;
    lds = std::max(lds, lds_bytes(t, W, t->tiles_per_wave, a.xs_cols, B, false));
    if (a.n_sg > 1) {
      a.partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + woff[i]);
      const uint32_t j = ra.nt++;
      ra.partials[j] = a.partials;
      ra.scales[j] = a.scales;
      ra.y[j] = ys[i];
      ra.rows[j] = a.rows;
      ra.n_sg[j] = a.n_sg;
      ra.row_begin[j] = red_rows;
      red_rows += a.rows;
    }
    ++ka.nt;
  }
  if (ka.nt == 0) return ECW_OK;
  ka.n_blocks = blocks;
  KernelFn fn = B == 1 ? pick_kernel<1, false>(ts[0]->coding) : pick_kernel<4, false>(ts[0]->coding);
  if (!fn) return fail(ECW_E_UNSUPPORTED, "no kernel for this payload / code width");
  if (lds > 160 * 1024) return fail(ECW_E_UNSUPPORTED, "launch shape needs more than 160 KiB of LDS");
  if (!lds_attribute_set(fn)) return fail(ECW_E_HIP, "hipFuncSetAttribute failed");
  const uint32_t grid = (blocks + 7) / 8 * 8;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(W * 64), (size_t)lds, (hipStream_t)stream, ka);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(ECW_E_HIP, std::string("launch failed: ") + hipGetErrorString(err));
  if (ra.nt) {
    ra.nb = (uint32_t)batch;
    ra.unit_scale = ts[0]->coding.payload == ECW_P_BF16_EXP;
    ra.total_rows = red_rows;
    const dim3 rgrid((red_rows + 255) / 256);
    if (B == 1)
      hipLaunchKernelGGL(k_reduce<1>, rgrid, dim3(256), 0, (hipStream_t)stream, ra);
    else
      hipLaunchKernelGGL(k_reduce<4>, rgrid, dim3(256), 0, (hipStream_t)stream, ra);
    err = hipGetLastError();
    if (err != hipSuccess) return fail(ECW_E_HIP, std::string("launch failed: ") + hipGetErrorString(err));
  }
  return ECW_OK;
}

}  // namespace ecw

using namespace ecw;

extern "C" ecw_status dec_gemv(ecw_stream stream, const ecw_tensor* t, const void* x, int x_dtype,
                               float* y, int batch, void* workspace, size_t ws_bytes) {
  clear_error();
  return launch_group(stream, &t, 1, x, x_dtype, &y, batch, workspace, ws_bytes);
}

extern "C" ecw_status dec_gemv_group_workspace_size(const ecw_tensor* const* t, int n, int batch,
                                                    size_t* bytes) {
  clear_error();
  if (!t || !bytes || n < 1 || n > kMaxGroup) return fail(ECW_E_INVALID_ARG, "bad arguments");
  if (batch < 1 || batch > 4) return fail(ECW_E_INVALID_ARG, "batch must be 1..4");
  for (int i = 0; i < n; ++i)
    if (!t[i] || t[i]->waves_per_block < 1 || t[i]->waves_per_block > 16 || t[i]->tiles_per_wave < 1)
      return fail(ECW_E_INVALID_ARG, "bad tensor or launch shape");
  *bytes = (size_t)group_workspace(t, n, batch, nullptr);
  return ECW_OK;
}

extern "C" ecw_status dec_gemv_group(ecw_stream stream, const ecw_tensor* const* t, int n, const void* x,
                                     int x_dtype, float* const* y, int batch, void* workspace,
                                     size_t ws_bytes) {
  clear_error();
  return launch_group(stream, t, n, x, x_dtype, y, batch, workspace, ws_bytes);
}

extern "C" ecw_status dec_materialize(ecw_stream stream, const ecw_tensor* t, uint16_t* symbols,
                                      void* w_out, uint32_t* tile_status) {
  clear_error();
  ecw_status st = check_tensor(t);
  if (st != ECW_OK) return st;
  if (t->n_tiles == 0) return ECW_OK;
  KArgs ka{};
  TArgs& a = ka.t[0];
  fill_tensor(t, a);
  a.sym_out = symbols;
  a.w_out = w_out;
  a.status_out = tile_status;
  a.nb = 1;
  a.tiles_per_wave = 1;   // every tile restarts its stream: per-tile status is exact
  const uint32_t W = std::min<uint32_t>(8, t->n_slices);
  a.n_sg = (t->n_slices + W - 1) / W;
  a.n_blocks = a.n_rg * a.n_sg;
  a.xs_cols = 0;
  ka.nt = 1;
  ka.n_blocks = a.n_blocks;
  KernelFn fn = pick_kernel<1, true>(t->coding);
  if (!fn) return fail(ECW_E_UNSUPPORTED, "no kernel for this payload / code width");
  const uint64_t lds = lds_bytes(t, W, 1, 0, 1, true);
  if (lds > 160 * 1024) return fail(ECW_E_UNSUPPORTED, "decode table needs more than 160 KiB of LDS");
  if (!lds_attribute_set(fn)) return fail(ECW_E_HIP, "hipFuncSetAttribute failed");
  const uint32_t grid = (ka.n_blocks + 7) / 8 * 8;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(W * 64), (size_t)lds, (hipStream_t)stream, ka);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(ECW_E_HIP, std::string("launch failed: ") + hipGetErrorString(err));
  return ECW_OK;
}
