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
// the same 64 rows and are summed in LDS in wave order.  When a row group spans
// several blocks, each block publishes its partial sums and takes a ticket; the
// block that arrives last adds all partials in block order.  Both orders are fixed,
// so results do not depend on scheduling.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <unordered_set>

#include "ecw_internal.h"

namespace ecw {

constexpr uint32_t kChunk = 256;           // words per chunk = 64 lanes x 8 bytes
constexpr uint32_t kRing = 512;            // words per wave ring (two chunks)
constexpr uint32_t kMirror = 64;           // copy of the ring head for reads that wrap
constexpr uint32_t kRingStride = kRing + kMirror;   // 1152 bytes per stream
constexpr uint32_t kPairTableBytes = 2048; // 256 symbols x up to 8 bytes
// BF16 raw-byte groups of the next 16 steps are loaded after the refill of this
// quarter of the current 16 steps, i.e. 8 steps before their first use.  Vector
// loads complete in order, and the refill's wait for its prefetched chunk is a wait
// for every load in flight (the compiler cannot count loads issued under
// data-dependent conditions).  Raw groups issued at the top of the 16 steps made
// every refill that followed soon after wait for them; issued here, only the last
// quarter's refill does.
constexpr int kRawQuarter = 2;

constexpr int kMaxGroup = 8;

// Payloads whose symbols carry several codes are multiplied with packed 16-bit dot
// products.  With fp16 activations and two codes per symbol the pair comes from the
// table entry itself (the high bytes of both codes' fp16 values); otherwise the
// entry's payload byte is the symbol and a 256-entry side table in LDS maps it to
// its codes as 16-bit floats of the activations' type.
template <int PAY, int KW>
constexpr bool kDot = PAY == 1 && KW >= 2;
template <int PAY, int KW, bool XBF>
constexpr bool kPairTable = PAY == 1 && (KW == 4 || (KW == 2 && XBF));
// BF16 weights with bf16 activations: two steps' weights are joined into one packed
// bf16 pair and multiplied with one bf16 dot product.
template <int PAY, int KW, bool XBF>
constexpr bool kBfPair = PAY == 2 && KW == 1 && XBF;
// BF16 exponent pairs: one symbol carries the exponents of two adjacent weights (the
// entry's high half holds both, rotated); escaped weights come from the tile's
// correction stream.
template <int PAY, int KW>
constexpr bool kBfSym2 = PAY == 2 && KW == 2;
// Quads of 4-bit codes over a table of stored 4-tuples: the entry's high half is the
// byte offset of the symbol's four codes in a per-block LDS table (two packed 16-bit
// pairs of the activations' type); escaped codes come from the tile's correction
// stream.
template <int PAY, int CB, int KW>
constexpr bool kQuad = PAY == 1 && CB == 4 && KW == 4;
// INT quads multiplied with fp16 activations (fused GEMV): the blob's decode entries
// are {f | bias << 16, the high bytes of the fp16 values of the stored tuple's four
// codes}, so a step reads one table entry and rebuilds both fp16 code pairs with byte
// permutes (an integer code |q| <= 8 has an fp16 value whose low byte is zero); the
// table is staged as it is stored.  The other INT quad decoders turn the entries back
// into symbol form in the prologue and read a tuple-indexed table.
template <int PAY, int CB, int KW, bool MAT, bool XBF>
constexpr bool kQuadF = kQuad<PAY, CB, KW> && !MAT && !XBF;
// Table entries whose high word is the bias alone (no payload bits beside it).
template <int PAY, int CB, int KW>
constexpr bool kCleanBias = (PAY == 1 && KW == 4 && CB != 4) || (PAY == 2 && KW == 1) || PAY == 4;

#define ECW_LDS __attribute__((address_space(3)))
template <typename T>
__device__ __forceinline__ ECW_LDS T* lds_ptr(uint32_t addr) {
  return (ECW_LDS T*)(size_t)addr;
}
// 8- and 16-byte LDS accesses (clang vector types: HIP's vector classes cannot be
// addressed in LDS address space)
typedef uint32_t ecw_u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t ecw_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_load2(uint32_t addr) {
  const ecw_u32x2 v = *lds_ptr<const ecw_u32x2>(addr);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint4 lds_load4(uint32_t addr) {
  const ecw_u32x4 v = *lds_ptr<const ecw_u32x4>(addr);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void lds_store2(uint32_t addr, uint2 v) {
  *lds_ptr<ecw_u32x2>(addr) = ecw_u32x2{v.x, v.y};
}
__device__ __forceinline__ void lds_store4(uint32_t addr, uint4 v) {
  *lds_ptr<ecw_u32x4>(addr) = ecw_u32x4{v.x, v.y, v.z, v.w};
}

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
  float* partials;          // [n_rg][n_sg][B][64] per-block sums (row groups over several blocks)
  uint32_t* tickets;        // [n_rg] arrival counters, zero between calls
  uint16_t* sym_out;
  void* w_out;
  uint32_t* status_out;
  void* deq_out;            // dequantised weights [rows][cols], fp16 or bf16 (decode-only)
  uint32_t deq_bf16;
  uint32_t rows, cols, n_rg, n_sl, s_full, s_last, log2m, tile_cols;
  uint32_t tiles_per_wave, n_sg, n_blocks, syms_per_row;
  uint32_t x_is_bf16, nb, lut_entries, xs_cols, ns, rpb;
  uint32_t raw_full_bytes, raw_rg_bytes;
  const uint8_t* tables;   // TABLES section (E8 decode-only hook: value offsets; INT quads: stored tuples)
  uint32_t quad_t;         // INT quads: stored tuples (entries of the LDS tuple table), else 0
};

// Launch arguments.  The fields a block needs to find its tensor are also passed as
// the kernel's leading scalar arguments, which the build preloads into scalar
// registers at wave launch (kernel-argument preloading of gfx950): a block finds its
// tensor without a memory round trip, and only the tensor's own fields are loaded.
// The launch shape is passed here instead of being read from the dispatch packet.
struct KArgs {
  uint32_t n_blocks;                 // total logical blocks
  uint32_t nt;                       // tensors in the launch
  uint32_t waves;                    // waves per block (blockDim.x / 64)
  uint32_t grid;                     // blocks launched (a multiple of 8)
  uint32_t block_begin[kMaxGroup];   // first logical block of each tensor
  TArgs t[kMaxGroup];
};

// x' = f * (x >> m) + bias in one v_mad_u32_u24 (both factors < 2^24; the payload
// byte in bits 24..31 of the table word is ignored by the 24-bit multiply).
__device__ __forceinline__ uint32_t mad_u24(uint32_t a, uint32_t b, uint32_t c) {
  return __umul24(a, b) + c;
}

// acc + f16(h >> 16) * x in fp32 (v_fma_mix_f32: operand 0 is the fp16 in the high
// half of h, operands 1 and 2 are fp32).  Exact widening of the fp16 weight.
__device__ __forceinline__ float fma_mix_hi(uint32_t h, float x, float acc) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "=v"(d) : "v"(h), "v"(x), "v"(acc));
  return d;
}

typedef _Float16 ecw_half2 __attribute__((ext_vector_type(2)));
typedef short ecw_short2 __attribute__((ext_vector_type(2)));

// acc + w.lo * x.lo + w.hi * x.hi, 16-bit operands (fp16 or bf16), fp32 accumulate.
template <bool XBF>
__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
  if constexpr (XBF)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(ecw_short2, w), __builtin_bit_cast(ecw_short2, x),
                                           acc, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(ecw_half2, w), __builtin_bit_cast(ecw_half2, x), acc, false);
}

// x = (x << 16) | w on the lanes of `mask` only (exec-masked v_lshl_or).  Inline asm
// so the update stays one VALU op under a scalar exec swap instead of a select.
__device__ __forceinline__ uint32_t shift_in(uint64_t mask, uint32_t x, uint32_t w) {
  uint64_t save;
  asm("s_and_saveexec_b64 %1, %2\n\tv_lshl_or_b32 %0, %0, 16, %3\n\ts_mov_b64 exec, %1"
      : "+v"(x), "=&s"(save) : "s"(mask), "v"(w) : "scc");
  return x;
}

// Pins a value at this point of the instruction stream: the multiply-adds of a step
// are then issued with the step instead of being sunk to the end of the unrolled
// loop, which would keep every step's table entry live (and spill).
template <int B>
__device__ __forceinline__ void pin(float* acc) {
#pragma unroll
  for (int b = 0; b < B; ++b) asm volatile("" : "+v"(acc[b]));
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// ---- the per-stream pieces of one decode step (scalar state, kept in registers)

// A4: one symbol decode.  Returns the table entry (f | a8 << 24, bias [| h16 << 16]).
template <bool CLEAN>
__device__ __forceinline__ uint2 decode_step(uint32_t& x, uint32_t lut, uint32_t m, uint32_t mmask) {
  const uint2 e = lds_load2(lut + ((x & mmask) << 3));
  x = mad_u24(x >> m, e.x, CLEAN ? e.y : (e.y & 0xFFFFu));
  return e;
}

// A4 for the INT quad entries as stored: x = f * (x >> m) + bias with f and bias the
// two halves of the entry's low word, taken by sub-dword operand selection (two VALU
// operations, as for the plain entries' mask and multiply-add).
__device__ __forceinline__ uint2 decode_step_q(uint32_t& x, uint32_t lut, uint32_t m, uint32_t mmask) {
  const uint2 e = lds_load2(lut + ((x & mmask) << 3));
  const uint32_t xs = x >> m;
  uint32_t r;
  asm("v_mul_u32_u24_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_0 src1_sel:DWORD\n\t"
      "v_add_u32_sdwa %0, %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1"
      : "=&v"(r) : "v"(e.x), "v"(xs));
  x = r;
  return e;
}

// A5: renormalise the wave's 64 states against the stream's LDS ring.  Every lane
// reads the word at its prefix offset (always inside the ring plus its mirror) and
// keeps it only if it needs one.  rposb: read position in bytes.
template <bool RAGGED>
__device__ __forceinline__ void renorm_step(uint32_t& x, uint32_t& rposb, uint32_t ring, bool active) {
  uint64_t msk;
  if constexpr (RAGGED)
    msk = __ballot(active && (x < kStateL));
  else
    msk = __builtin_amdgcn_ballot_w64(x < kStateL);
  const uint32_t base = ring + (rposb & (2 * kRing - 2));
  const uint32_t w = *lds_ptr<const uint16_t>(base + (lanes_below(msk) << 1));
  x = shift_in(msk, x, w);
  // rposb += 2 * popcount(mask) as one scalar op (kept opaque so the compiler does
  // not rebuild the pointer from a running count every step)
  const uint32_t cnt = (uint32_t)__popcll(msk);
  asm("s_lshl1_add_u32 %0, %1, %0" : "+s"(rposb) : "s"(cnt) : "scc");
}

// The same step split in two halves, so that two streams issue both ring reads
// before either waits (the exec-masked shift is an asm block, which the compiler
// does not move loads across).
struct RenormRead {
  uint64_t mask;
  uint32_t w;
};

template <bool RAGGED>
__device__ __forceinline__ RenormRead renorm_read(uint32_t x, uint32_t rposb, uint32_t ring, bool active) {
  RenormRead r;
  if constexpr (RAGGED)
    r.mask = __ballot(active && (x < kStateL));
  else
    r.mask = __builtin_amdgcn_ballot_w64(x < kStateL);
  const uint32_t base = ring + (rposb & (2 * kRing - 2));
  r.w = *lds_ptr<const uint16_t>(base + (lanes_below(r.mask) << 1));
  return r;
}

// Both streams' shifts in one asm block: its inputs are both ring words, so the
// two ring reads are issued before the first wait.
__device__ __forceinline__ void renorm_apply2(const RenormRead& ra, uint32_t& xa, uint32_t& rposa,
                                              const RenormRead& rb, uint32_t& xb, uint32_t& rposb) {
  uint64_t save;
  asm("s_and_saveexec_b64 %2, %3\n\tv_lshl_or_b32 %0, %0, 16, %4\n\ts_mov_b64 exec, %2\n\t"
      "s_and_saveexec_b64 %2, %5\n\tv_lshl_or_b32 %1, %1, 16, %6\n\ts_mov_b64 exec, %2"
      : "+v"(xa), "+v"(xb), "=&s"(save) : "s"(ra.mask), "v"(ra.w), "s"(rb.mask), "v"(rb.w) : "scc");
  const uint32_t ca = (uint32_t)__popcll(ra.mask), cb = (uint32_t)__popcll(rb.mask);
  asm("s_lshl1_add_u32 %0, %2, %0\n\ts_lshl1_add_u32 %1, %3, %1" : "+s"(rposa), "+s"(rposb) : "s"(ca), "s"(cb)
      : "scc");
}

// Keep the next four steps' reads inside committed ring data: commit the chunk held
// in `pre` when fewer than 256 words are ahead of the read position, and load the
// next one into `pre` (one chunk of prefetch distance).  wl: this lane's byte
// address in the stream's ring (ring + 8 * lane); src: the stream's first chunk
// (wave-uniform).
__device__ __forceinline__ void refill(uint32_t rposb, uint32_t& haveb, uint32_t& nc, uint2& pre, uint32_t wl,
                                       const uint2* src, uint32_t nch, uint32_t lane) {
  if (rposb + 8 * 64 > haveb) {      // wave-uniform
    if (nc & 1u) {
      lds_store2(wl + 2 * kChunk, pre);
    } else {
      lds_store2(wl, pre);
      if (lane < 16) lds_store2(wl + 2 * kRing, pre);
    }
    haveb += 2 * kChunk;
    ++nc;
    if (nc < nch) pre = src[(uint64_t)nc * 64 + lane];
  }
}

// a * b in fp32, kept a separate multiply: fused with a following conversion to fp16
// the compiler emits a mixed multiply-add with a +0.0 addend, which turns a product
// of -0.0 into +0.0
__device__ __forceinline__ float exact_product(float a, float b) {
  float p = a * b;
  asm volatile("" : "+v"(p));
  return p;
}

// Correction stream of a BF16 exponent-pair or INT quad tile (MINE page, Section 4.1
// "Escapes": escaped weights were coded as 0; their records follow the tile's ANS
// words).
// After the tile's last symbol: every lane reads its bit of the 64-bit lane mask,
// then the lanes that still hold records read one each per round, at their prefix
// offset among those lanes (the renormalisation's coordination), and add weight *
// activation (OUT = kOutAcc), or store the weight (kOutBits: the bf16 bits into
// w_out; kOutCode: the int8 code into w_out; kOutF16 / kOutBf16: the value, times
// the row scale with SC, into deq_out).  Rounds end when every lane
// has read its row's last record, or after `width` rounds (a row has at most
// `width` escapes) so that a damaged stream still ends.  The general rounds read a
// record as two 16-bit halves, each wrapped into the ring (the fused product's own
// rounds are described there).  col: staged column of the tile's first
// weight; width: weights per row in the tile; wrow: output index of this row's first
// weight in the tile.
constexpr int kOutAcc = 0, kOutBits = 1, kOutF16 = 2, kOutBf16 = 3, kOutCode = 4;

// fp32 -> 16-bit float bits, round to nearest even (bf16: finite inputs)
template <bool OBF>
__device__ __forceinline__ uint32_t to16(float v) {
  if constexpr (OBF) {
    const uint32_t b = __float_as_uint(v);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
  } else {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v);
  }
}

// SC: the dense outputs are the record's value times the row scale (INT quads).
// PKX: activations staged as packed 16-bit pairs [column / 2][B] of the type XBF
// selects (else fp32 [column][B]).
template <int B, int OUT, bool XBF, bool SC = false, bool PKX = XBF>
__device__ __forceinline__ void tile_corrections(const TArgs& a, uint32_t& rposb, uint32_t& haveb, uint32_t& nc,
                                              uint2& pre, uint32_t wl, const uint2* src, uint32_t nch,
                                              uint32_t lane, uint32_t ring, uint32_t xs, uint32_t col,
                                              uint32_t width, bool active, uint64_t wrow, float* acc,
                                              float scale = 1.f) {
  constexpr uint32_t kWrap = 2 * kRing - 2;
  refill(rposb, haveb, nc, pre, wl, src, nch, lane);
  const uint32_t mw = *lds_ptr<const uint16_t>(ring + ((rposb + 2 * (lane >> 4)) & kWrap));
  bool has = active && ((mw >> (lane & 15)) & 1u);
  rposb += 2 * kEscMaskWords;
  uint64_t act = __ballot(has);
  if constexpr (OUT == kOutAcc) {
    // The fused product's rounds, written for few instructions (the launches are
    // issue-bound): both halves of a record from one ring address (a record that
    // starts on the ring's last word reads its high half from the mirror of the ring
    // head), the column clamped into the tile instead of an exec branch, the
    // activation read as one 16-bit value, and the multiply-add kept by a select.
    // The same multiply-adds in the same order as the general rounds below.
    const uint32_t wmax = width - 1;
    for (uint32_t round = 0; act != 0 && round < width; ++round) {
      refill(rposb, haveb, nc, pre, wl, src, nch, lane);
      const uint32_t ra = ring + ((rposb + 4 * lanes_below(act)) & kWrap);
      const uint32_t rec = (uint32_t)*lds_ptr<const uint16_t>(ra) |
                           ((uint32_t)*lds_ptr<const uint16_t>(ra + 2) << 16);
      rposb += 4 * (uint32_t)__popcll(act);
      const uint32_t c = (rec >> 16) & 0x7FFu;
      const bool use = has && c < width;
      const uint32_t cx = col + (c < wmax ? c : wmax);
      const float w = __uint_as_float(rec << 16);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        float xv;
        if constexpr (PKX) {
          // packed pairs [column / 2][B]; the tile starts on an even column
          const uint32_t h = *lds_ptr<const uint16_t>(xs + ((cx >> 1) * B + b) * 4 + (cx & 1u) * 2);
          xv = XBF ? __uint_as_float(h << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)h);
        } else {
          xv = *lds_ptr<const float>(xs + (cx * B + b) * 4);
        }
        const float f = fmaf(w, xv, acc[b]);
        acc[b] = use ? f : acc[b];
      }
      has = has && !(rec & kEscLast);
      act = __ballot(has);
    }
  } else {
    // the general rounds: the decode-only hook and the dequantising decode store
    // each escaped weight
    for (uint32_t round = 0; act != 0 && round < width; ++round) {
      refill(rposb, haveb, nc, pre, wl, src, nch, lane);
      const uint32_t pos = rposb + 4 * lanes_below(act);
      const uint32_t lo = *lds_ptr<const uint16_t>(ring + (pos & kWrap));
      const uint32_t hi = *lds_ptr<const uint16_t>(ring + ((pos + 2) & kWrap));
      rposb += 4 * (uint32_t)__popcll(act);
      if (has) {
        const uint32_t rec = lo | (hi << 16);
        const uint32_t c = (rec >> 16) & 0x7FFu;
        if (c < width) {
          if constexpr (OUT == kOutBits) {
            if (a.w_out) static_cast<uint16_t*>(a.w_out)[wrow + c] = (uint16_t)rec;
          } else if constexpr (OUT == kOutCode) {
            if (a.w_out) static_cast<int8_t*>(a.w_out)[wrow + c] = (int8_t)(int)__uint_as_float(rec << 16);
          } else if constexpr (OUT == kOutBf16 && !SC) {
            static_cast<uint16_t*>(a.deq_out)[wrow + c] = (uint16_t)rec;
          } else {
            static_assert(OUT == kOutBf16 || OUT == kOutF16, "unknown correction output");
            float v = __uint_as_float(rec << 16);
            if constexpr (SC) v = exact_product(v, scale);
            static_cast<uint16_t*>(a.deq_out)[wrow + c] = (uint16_t)to16<OUT == kOutBf16>(v);
          }
        }
        if (rec & kEscLast) has = false;
      }
      act = __ballot(has);
    }
  }
}

// BF16 join from whole bytes (DFloat11 page, Algorithm 1: the decoded exponent
// joined with the stored sign and mantissa).  The table byte a8 holds the exponent
// rotated right by one bit; the raw byte r is sign << 7 | mantissa.  The bf16 high
// byte is sign | a8[6:0] and its low byte a8[7] | mantissa, so two byte permutes and
// one bit-field select build it.  Selector bytes index {src0: bytes 4-7, src1: 0-3};
// 0x0C yields zero.
//   bf16_in_f32: one weight as fp32 bits (bf16 in the high half); e.x holds a8 in
//   byte 3, rdw holds r in byte q.
__device__ __forceinline__ uint32_t bf16_in_f32(uint32_t ex, uint32_t rdw, int q) {
  const uint32_t p1 = __builtin_amdgcn_perm(ex, rdw, 0x07000C0Cu | ((uint32_t)q << 16));   // [0, 0, r, a8]
  const uint32_t p2 = __builtin_amdgcn_perm(ex, rdw, 0x00070C0Cu | ((uint32_t)q << 24));   // [0, 0, a8, r]
  return (p2 & 0x80800000u) | (p1 & 0x7F7F7F7Fu);
}
//   bf16_pair: the weights of two consecutive steps (first in the low half); their
//   raw bytes are bytes q and q + 1 of rdw.
__device__ __forceinline__ uint32_t bf16_pair(uint32_t ex0, uint32_t ex1, uint32_t rdw, int q) {
  const uint32_t a = __builtin_amdgcn_perm(ex1, ex0, 0x0C0C0703u);                           // [a8_0, a8_1, 0, 0]
  const uint32_t qq = (uint32_t)q;
  const uint32_t p1 = __builtin_amdgcn_perm(a, rdw, qq | (4u << 8) | ((qq + 1) << 16) | (5u << 24));
  const uint32_t p2 = __builtin_amdgcn_perm(a, rdw, 4u | (qq << 8) | (5u << 16) | ((qq + 1) << 24));
  return (p2 & 0x80808080u) | (p1 & 0x7F7F7F7Fu);
}

//   bf16_sym2: both weights of a BF16 exponent-pair symbol (first in the low half)
//   from the entry's high word (bias | rot e0 << 16 | rot e1 << 24) and their raw
//   bytes, bytes q and q + 1 of rdw.
__device__ __forceinline__ uint32_t bf16_sym2(uint32_t ey, uint32_t rdw, int q) {
  const uint32_t qq = (uint32_t)q;
  const uint32_t p1 = __builtin_amdgcn_perm(ey, rdw, qq | (6u << 8) | ((qq + 1) << 16) | (7u << 24));
  const uint32_t p2 = __builtin_amdgcn_perm(ey, rdw, 6u | (qq << 8) | (7u << 16) | ((qq + 1) << 24));
  return (p2 & 0x80808080u) | (p1 & 0x7F7F7F7Fu);
}

// Activations of four bf16-pair steps: two pair words per batch row, staged as
// [pair word][B].
template <int B>
__device__ __forceinline__ void bf16_pair_x(uint32_t addr, uint32_t* xp) {
  if constexpr (B == 1) {
    const uint2 v = lds_load2(addr);
    xp[0] = v.x;
    xp[1] = v.y;
  } else {
    const uint4 v0 = lds_load4(addr), v1 = lds_load4(addr + 16);
    xp[0] = v0.x; xp[1] = v0.y; xp[2] = v0.z; xp[3] = v0.w;
    xp[4] = v1.x; xp[5] = v1.y; xp[6] = v1.z; xp[7] = v1.w;
  }
}

// A6 + A7: rebuild the weight(s) of one symbol in registers and accumulate.
// xw: this symbol's activations as 32-bit words (fp32 [KW][B], or for the dot path
// packed 16-bit pairs [KW/2][B]).  BF16: rdw is the raw dword holding this step's
// byte, at byte q.
template <int PAY, int CB, int KW, int B, bool XBF>
__device__ __forceinline__ void mac(const uint2 e, const uint32_t* xw, uint32_t rdw, int q, float* acc) {
  static_assert(!kQuad<PAY, CB, KW>, "INT quads multiply in wave_body, after the renormalisation");
  if constexpr (kDot<PAY, KW> && !kPairTable<PAY, KW, XBF>) {
    // fp16 (q0, q1) = bytes (0, hi8 q0, 0, hi8 q1) from the entry's high half
    const uint32_t wp = __builtin_amdgcn_perm(e.y, e.y, 0x030C020Cu);
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = dot2<false>(wp, xw[b], acc[b]);
  } else if constexpr (kDot<PAY, KW>) {
    // pair table at LDS address 0: entry of symbol s at s * 4 (KW 2) or s * 8 (KW 4);
    // bits 22..23 of e.x are zero because f < 2^14
    if constexpr (KW == 2) {
      const uint32_t wp = *lds_ptr<const uint32_t>(e.x >> 22);
#pragma unroll
      for (int b = 0; b < B; ++b) acc[b] = dot2<XBF>(wp, xw[b], acc[b]);
    } else {
      const uint2 wp = lds_load2(e.x >> 21);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        acc[b] = dot2<XBF>(wp.x, xw[b], acc[b]);
        acc[b] = dot2<XBF>(wp.y, xw[B + b], acc[b]);
      }
    }
  } else if constexpr (PAY == 1) {
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = fma_mix_hi(e.y, __uint_as_float(xw[b]), acc[b]);   // q0
  } else if constexpr (kBfSym2<PAY, KW>) {
    const uint32_t wp = bf16_sym2(e.y, rdw, q);
    if constexpr (XBF) {
#pragma unroll
      for (int b = 0; b < B; ++b) acc[b] = dot2<true>(wp, xw[b], acc[b]);
    } else {
      const float w0 = __uint_as_float(wp << 16), w1 = __uint_as_float(wp & 0xFFFF0000u);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        acc[b] = fmaf(w0, __uint_as_float(xw[b]), acc[b]);
        acc[b] = fmaf(w1, __uint_as_float(xw[B + b]), acc[b]);
      }
    }
  } else if constexpr (PAY == 2) {
    const float w = __uint_as_float(bf16_in_f32(e.x, rdw, q));
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = fmaf(w, __uint_as_float(xw[b]), acc[b]);
  } else {
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = fma_mix_hi(e.y, __uint_as_float(xw[b]), acc[b]);   // e4m3 value
  }
}

__device__ __forceinline__ uint32_t raw_dword(const uint4& g, int u) {
  return (u < 4) ? g.x : (u < 8) ? g.y : (u < 12) ? g.z : g.w;
}
__device__ __forceinline__ uint32_t raw_byte(const uint4& g, int u) {
  return (raw_dword(g, u) >> (8 * (u & 3))) & 0xFFu;
}

__device__ __forceinline__ const uint8_t* raw_tile(const TArgs& a, uint32_t rg, uint32_t sl, uint32_t lane) {
  return a.raw + (uint64_t)rg * a.raw_rg_bytes + (uint64_t)sl * a.raw_full_bytes + lane * 16;
}

// Wave priority by the work a wave has left in its tile: `left` of `total` steps (or
// lattice blocks), four levels by quarter.  Blocks sharing a CU start about a
// microsecond apart and the later one stages its tables more slowly while the first
// decodes; left alone it ends long after, with its CU half empty.  Waves with more
// work left take issue slots first, so the blocks of a CU end closer together.
// Kernels enter at the top level, so a late block's staging is not held back either.
__device__ __forceinline__ void prio_by_work_left(uint32_t left, uint32_t total) {
  const uint32_t q = total >> 2;
  if (left > total - q) __builtin_amdgcn_s_setprio(3);
  else if (left > 2 * q) __builtin_amdgcn_s_setprio(2);
  else if (left > q) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Start of a wave's word stream over tiles [t0, t1): chunk-aligned word start gb,
// chunk count nch, first read position rposb (bytes from gb), the first tile's
// start state, the first two chunks and the one-ahead prefetch.  Filled in two
// phases so the loads overlap the block's table staging: head_begin issues the
// tile offsets and start state, head_chunks (after staging, before the barrier)
// the first chunk loads.
struct StreamHead {
  uint32_t gb, nch, rposb, st;
  uint2 c0, c1, pre;
  const uint2* src;
};

__device__ __forceinline__ void head_begin(const TArgs& a, uint32_t t0, uint32_t t1, uint32_t lane, StreamHead& h) {
  h.gb = 0;          // word offset of t0 until head_chunks
  h.nch = 0;         // word offset of t1 until head_chunks
  h.st = kStateL;
  if (t0 < t1) {
    h.gb = a.offsets[t0];
    h.nch = a.offsets[t1];
    h.st = a.states[(uint64_t)t0 * 64 + lane];
  }
}

__device__ __forceinline__ void head_chunks(const TArgs& a, uint32_t lane, StreamHead& h) {
  const uint32_t wb = h.gb, we = h.nch;
  h.gb = wb & ~(kChunk - 1);
  h.nch = (we - h.gb + kChunk - 1) / kChunk;
  h.rposb = (wb - h.gb) * 2;
  h.src = reinterpret_cast<const uint2*>(a.words + h.gb);
  const uint2 zero2 = {0u, 0u};
  h.c0 = h.nch > 0 ? h.src[lane] : zero2;
  h.c1 = h.nch > 1 ? h.src[64 + lane] : zero2;
  h.pre = h.nch > 2 ? h.src[128 + lane] : zero2;
}

// First two chunks into the ring (and the head mirror); after the block barrier.
// wl: ring + 8 * lane.
__device__ __forceinline__ void head_ring(const StreamHead& h, uint32_t wl, uint32_t lane) {
  lds_store2(wl, h.c0);
  if (lane < 16) lds_store2(wl + 2 * kRing, h.c0);
  lds_store2(wl + 2 * kChunk, h.c1);
}

// The wave body: the wave's tiles [t0, t1) (consecutive slices of one row group)
// are decoded as one stream of words; each tile starts from its own states.
// MAT: decode-only test hook.  ring: LDS byte address of the wave's ring.  xs: LDS
// byte address of the staged activations.
template <int PAY, int CB, int KW, int B, bool MAT, bool RAGGED, bool XBF>
__device__ __forceinline__ void wave_body(const TArgs& a, const StreamHead& h, uint32_t lut, uint32_t xs,
                                          uint32_t ring, uint32_t rg, uint32_t t0, uint32_t t1, uint32_t c_lo,
                                          uint32_t lane, bool active, float* acc) {
  constexpr int U = 16;
  constexpr bool BF2 = kBfSym2<PAY, KW>;               // bf16 exponent-pair symbols
  constexpr bool QD = kQuad<PAY, CB, KW>;              // INT quads over stored tuples
  constexpr bool QF = kQuadF<PAY, CB, KW, MAT, XBF>;    // ... codes in the entries (fp16 x)
  constexpr bool DOT = kDot<PAY, KW> || (BF2 && XBF);
  constexpr bool BFP = kBfPair<PAY, KW, XBF> && !MAT;   // bf16 weight pairs, two steps per dot
  constexpr int RG = BF2 ? 2 : 1;                      // raw 16-byte groups per U steps
  constexpr bool PK = DOT || BFP;                   // activations staged as 16-bit pairs
  constexpr bool CLEAN = kCleanBias<PAY, CB, KW>;
  constexpr int XW = DOT ? (KW / 2) * B : KW * B;   // 32-bit activation words per step
  const uint32_t m = a.log2m, mmask = (1u << m) - 1u;
  const uint32_t row = rg * 64 + lane;
  const uint32_t sl0 = rg * a.n_sl;
  const uint4 zero4 = {0u, 0u, 0u, 0u};

  const uint32_t wl = ring + lane * 8;
  head_ring(h, wl, lane);
  const uint32_t gb = h.gb, nch = h.nch;
  const uint2* src = h.src;
  uint32_t rposb = h.rposb;
  uint2 pre = h.pre;
  uint32_t haveb = 4 * kChunk, nc = 2;
  uint32_t st = h.st;
  // BF16 raw bytes: the groups of each U steps are loaded one U-step block ahead
  const uint8_t* rawp = raw_tile(a, rg, t0 - sl0, lane);
  uint4 rnext[RG];
#pragma unroll
  for (int i = 0; i < RG; ++i) rnext[i] = zero4;
  if constexpr (PAY == 2) {
#pragma unroll
    for (int i = 0; i < RG; ++i) rnext[i] = *reinterpret_cast<const uint4*>(rawp + 1024 * i);
  }

  for (uint32_t t = t0; t < t1; ++t) {
    uint32_t x = st;
    if (t + 1 < t1) st = a.states[(uint64_t)(t + 1) * 64 + lane];
    const uint32_t sl = t - sl0;
    const uint32_t S = (sl + 1 == a.n_sl) ? a.s_last : a.s_full;
    const uint32_t col = sl * a.tile_cols - c_lo;

    for (uint32_t j = 0; j < S; j += U) {
      prio_by_work_left(S - j, S);
      uint4 rgp[RG];
#pragma unroll
      for (int i = 0; i < RG; ++i) rgp[i] = zero4;
      bool more = false;            // raw groups of the next U steps to prefetch
      if constexpr (PAY == 2) {
#pragma unroll
        for (int i = 0; i < RG; ++i) rgp[i] = rnext[i];
        // the next groups: of this tile, else the first of the wave's next tile
        more = j + U < S || t + 1 < t1;                     // wave-uniform
        rawp = j + U < S ? rawp + 1024 * RG : raw_tile(a, rg, sl + 1, lane);
      }
      // activation words of step j: fp32 [col][B], or packed pairs [col / 2][B]
      const uint32_t xg = xs + ((col + KW * j) * B / (PK ? 2 : 1)) * 4;
#pragma unroll
      for (int qtr = 0; qtr < U / 4; ++qtr) {
        refill(rposb, haveb, nc, pre, wl, src, nch, lane);
        if constexpr (PAY == 2) {
          if (qtr == kRawQuarter && more) {
#pragma unroll
            for (int i = 0; i < RG; ++i) rnext[i] = *reinterpret_cast<const uint4*>(rawp + 1024 * i);
          }
        }
        uint4 xq[MAT || BFP ? 1 : XW];
        uint32_t xp[BFP ? 2 * B : 1];     // bf16 pairs: two pair words per batch row
        if constexpr (BFP) {
          bf16_pair_x<B>(xg + qtr * 8 * B, xp);
        } else if constexpr (!MAT) {
#pragma unroll
          for (int i = 0; i < XW; ++i) xq[i] = lds_load4(xg + (qtr * XW + i) * 16);
        }
        uint32_t ex0 = 0;                 // bf16 pairs: the first step's table word
        uint2 qwp = {0u, 0u};             // INT quads: this step's codes
#pragma unroll
        for (int u4 = 0; u4 < 4; ++u4) {
          const int u = qtr * 4 + u4;
          const uint32_t step = j + u;
          const uint2 e = QF ? decode_step_q(x, lut, m, mmask) : decode_step<CLEAN>(x, lut, m, mmask);
          // BF16: the dword of raw bytes holding this step's (first) weight, at byte q
          uint32_t rdw;
          int q;
          if constexpr (BF2) {
            rdw = raw_dword(rgp[u >> 3], (2 * u) & 15);
            q = (u & 1) * 2;
          } else {
            rdw = raw_dword(rgp[0], u);
            q = u & 3;
          }
          if constexpr (BFP) {
            if (u4 & 1) {
              const uint32_t wp = bf16_pair(ex0, e.x, rdw, (u - 1) & 3);
#pragma unroll
              for (int b = 0; b < B; ++b) acc[b] = dot2<true>(wp, xp[(u4 >> 1) * B + b], acc[b]);
              pin<B>(acc);
            } else {
              ex0 = e.x;
            }
          } else if constexpr (QF) {
            // the codes' fp16 pairs (q0, q1) and (q2, q3): bytes [0, hi8 q, 0, hi8 q']
            qwp.x = __builtin_amdgcn_perm(e.y, e.y, 0x010C000Cu);
            qwp.y = __builtin_amdgcn_perm(e.y, e.y, 0x030C020Cu);
          } else if constexpr (QD && !MAT) {
            qwp = lds_load2(e.y >> 16);     // multiplied after the renormalisation's ring read
          } else if constexpr (!MAT) {
            mac<PAY, CB, KW, B, XBF>(e, reinterpret_cast<const uint32_t*>(xq) + u4 * XW, rdw, q, acc);
            pin<B>(acc);
          } else if (!RAGGED || active) {
            uint32_t aux = e.x >> 24;
            if constexpr (PAY == 2 && !BF2) aux = ((aux << 1) | (aux >> 7)) & 0xFFu;   // rotated exponent
            uint32_t symbol = aux;
            if constexpr (QD) {
              symbol = e.y >> 19;                                   // index of the stored tuple
              aux = *lds_ptr<const uint32_t>(e.y >> 16);            // its codes' digits
            }
            int q[KW > 0 ? KW : 1];
            if constexpr (PAY == 1) {
              constexpr int half = 1 << (CB - 1);
              if constexpr (KW == 1) {
                q[0] = (int)(int8_t)aux;
                symbol = (uint32_t)(q[0] + half);
              } else {
#pragma unroll
                for (int i = 0; i < KW; ++i) q[i] = (int)((aux >> (CB * i)) & ((1u << CB) - 1)) - half;
              }
            }
            if (a.sym_out) a.sym_out[(uint64_t)row * a.syms_per_row + (uint64_t)sl * a.s_full + step] = (uint16_t)symbol;
            if (a.w_out) {
              const uint64_t wi = (uint64_t)row * a.cols + (uint64_t)sl * a.tile_cols + (uint64_t)step * KW;
              if constexpr (PAY == 1) {
#pragma unroll
                for (int i = 0; i < KW; ++i) static_cast<int8_t*>(a.w_out)[wi + i] = (int8_t)q[i];
              } else if constexpr (BF2) {
                // escaped weights are written here as +0.0 and overwritten by the
                // tile's correction stream
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                  const int byte = 2 * u + i;
                  const uint32_t r = raw_byte(rgp[byte >> 4], byte & 15);
                  const uint32_t ar = (e.y >> (16 + 8 * i)) & 0xFFu;
                  const uint32_t ex = ((ar << 1) | (ar >> 7)) & 0xFFu;
                  static_cast<uint16_t*>(a.w_out)[wi + i] = (uint16_t)(((r & 0x80u) << 8) | (ex << 7) | (r & 0x7Fu));
                }
              } else if constexpr (PAY == 2) {
                const uint32_t r = raw_byte(rgp[0], u);
                static_cast<uint16_t*>(a.w_out)[wi] = (uint16_t)(((r & 0x80u) << 8) | (aux << 7) | (r & 0x7Fu));
              } else {
                static_cast<uint8_t*>(a.w_out)[wi] = (uint8_t)aux;
              }
            }
          }
          renorm_step<RAGGED>(x, rposb, ring, active);
          if constexpr (QD && !MAT) {
            // the stored tuple's codes (two 16-bit pairs) times this step's activations;
            // their table read overlapped the ring read
            const uint32_t* xw = reinterpret_cast<const uint32_t*>(xq) + u4 * XW;
#pragma unroll
            for (int b = 0; b < B; ++b) {
              acc[b] = dot2<XBF>(qwp.x, xw[b], acc[b]);
              acc[b] = dot2<XBF>(qwp.y, xw[B + b], acc[b]);
            }
            pin<B>(acc);
          }
        }
      }
    }
    if constexpr (BF2 || QD)
      tile_corrections<B, MAT ? (QD ? kOutCode : kOutBits) : kOutAcc, XBF, false, PK>(
          a, rposb, haveb, nc, pre, wl, src, nch, lane, ring, xs, col, KW * S, active,
          (uint64_t)row * a.cols + (uint64_t)sl * a.tile_cols, acc);
    if constexpr (MAT) {
      const bool ok_lane = !active || x == kStateL;
      const uint64_t bad = __ballot(!ok_lane);
      if (lane == 0 && a.status_out)
        a.status_out[t] = (bad != 0 ? 1u : 0u) | ((rposb != (a.offsets[t + 1] - gb) * 2) ? 2u : 0u);
    }
  }
}

// Dequantising decode (decode-only, at full speed): the wave's tiles are decoded as
// in wave_body and every weight is rebuilt as its real value (INT: code * row scale;
// BF16: the bf16 value; FP8: the E4M3 value * row scale), each exact in fp32, then
// rounded to fp16 or bf16 (round to nearest even).  The output is the row-major
// matrix [rows][cols], written row-contiguous: every 32 weights (16 for one code per
// symbol) each lane puts its row's segment into a per-wave LDS tile [64 rows][pitch],
// and the wave writes the tile back four lanes per 64-byte row segment, so one store
// instruction covers 16 rows x 64 B instead of 64 scattered rows.  The stores are
// non-temporal (streamed past the caches: the dense matrix is read once, later, by
// the GEMM), measured 30% faster than plain stores for the INT4 gate tensor.  BF16 pairs then
// overwrite their escaped weights from the correction stream, after a wait for the
// tile's stores.  stage: LDS byte address of the wave's tile.
constexpr uint32_t kStagePitch = 80;       // 64 B of a row segment + 16 B against bank conflicts

template <int PAY, int CB, int KW>
constexpr int kFlushSteps = KW == 4 ? 8 : 16;   // 32 weights per flush (16 for KW = 1)

template <int PAY, int CB, int KW, bool RAGGED, bool OBF>
__device__ __forceinline__ void wave_body_deq(const TArgs& a, const StreamHead& h, uint32_t lut, uint32_t ring,
                                              uint32_t stage, uint32_t rg, uint32_t t0, uint32_t t1, uint32_t lane,
                                              bool active) {
  constexpr int U = 16;
  constexpr int FS = kFlushSteps<PAY, CB, KW>;
  constexpr int FW = FS * KW;                  // weights per lane per flush: 16 or 32
  constexpr int CPR = FW / 8;                  // 16-byte chunks per row segment: 2 or 4
  constexpr bool BF2 = kBfSym2<PAY, KW>;
  constexpr bool QD = kQuad<PAY, CB, KW>;
  constexpr bool CLEAN = kCleanBias<PAY, CB, KW>;
  constexpr int RG = BF2 ? 2 : 1;
  const uint32_t m = a.log2m, mmask = (1u << m) - 1u;
  const uint32_t row = rg * 64 + lane;
  const uint32_t sl0 = rg * a.n_sl;
  const uint4 zero4 = {0u, 0u, 0u, 0u};
  uint16_t* out = static_cast<uint16_t*>(a.deq_out);
  float scale = 1.f;
  if constexpr (PAY != 2) scale = active ? (float)__builtin_bit_cast(_Float16, a.scales[row]) : 0.f;

  const uint32_t wl = ring + lane * 8;
  head_ring(h, wl, lane);
  const uint32_t nch = h.nch;
  const uint2* src = h.src;
  uint32_t rposb = h.rposb;
  uint2 pre = h.pre;
  uint32_t haveb = 4 * kChunk, nc = 2;
  uint32_t st = h.st;
  const uint8_t* rawp = raw_tile(a, rg, t0 - sl0, lane);
  uint4 rnext[RG];
#pragma unroll
  for (int i = 0; i < RG; ++i) rnext[i] = zero4;
  if constexpr (PAY == 2) {
#pragma unroll
    for (int i = 0; i < RG; ++i) rnext[i] = *reinterpret_cast<const uint4*>(rawp + 1024 * i);
  }
  uint32_t pk[FW / 2];                         // this lane's segment, 16-bit values packed in pairs

  for (uint32_t t = t0; t < t1; ++t) {
    uint32_t x = st;
    if (t + 1 < t1) st = a.states[(uint64_t)(t + 1) * 64 + lane];
    const uint32_t sl = t - sl0;
    const uint32_t S = (sl + 1 == a.n_sl) ? a.s_last : a.s_full;
    const uint64_t colw = (uint64_t)sl * a.tile_cols;     // column of the tile's first weight

    for (uint32_t j = 0; j < S; j += U) {
      prio_by_work_left(S - j, S);
      uint4 rgp[RG];
#pragma unroll
      for (int i = 0; i < RG; ++i) rgp[i] = zero4;
      bool more = false;            // raw groups of the next U steps to prefetch
      if constexpr (PAY == 2) {
#pragma unroll
        for (int i = 0; i < RG; ++i) rgp[i] = rnext[i];
        more = j + U < S || t + 1 < t1;                     // wave-uniform
        rawp = j + U < S ? rawp + 1024 * RG : raw_tile(a, rg, sl + 1, lane);
      }
#pragma unroll
      for (int qtr = 0; qtr < U / 4; ++qtr) {
        refill(rposb, haveb, nc, pre, wl, src, nch, lane);
        if constexpr (PAY == 2) {
          if (qtr == kRawQuarter && more) {
#pragma unroll
            for (int i = 0; i < RG; ++i) rnext[i] = *reinterpret_cast<const uint4*>(rawp + 1024 * i);
          }
        }
#pragma unroll
        for (int u4 = 0; u4 < 4; ++u4) {
          const int u = qtr * 4 + u4;
          const uint2 e = QD ? decode_step_q(x, lut, m, mmask) : decode_step<CLEAN>(x, lut, m, mmask);
          uint32_t v[KW];                                   // this step's weights, 16-bit
          if constexpr (QD) {
            // INT quads: the codes' fp16 values, rebuilt from the entry's high bytes
            const uint32_t cp[2] = {__builtin_amdgcn_perm(e.y, e.y, 0x010C000Cu),
                                    __builtin_amdgcn_perm(e.y, e.y, 0x030C020Cu)};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float q = (float)__builtin_bit_cast(_Float16, (uint16_t)(cp[i >> 1] >> (16 * (i & 1))));
              v[i] = to16<OBF>(exact_product(q, scale));
            }
          } else if constexpr (PAY == 1) {
            const uint32_t aux = e.x >> 24;
            constexpr int half = 1 << (CB - 1);
#pragma unroll
            for (int i = 0; i < KW; ++i) {
              const int q = KW == 1 ? (int)(int8_t)aux : (int)((aux >> (CB * i)) & ((1u << CB) - 1)) - half;
              v[i] = to16<OBF>(exact_product((float)q, scale));
            }
          } else if constexpr (BF2) {
            const uint32_t wp = bf16_sym2(e.y, raw_dword(rgp[u >> 3], (2 * u) & 15), (u & 1) * 2);
            if constexpr (OBF) {
              v[0] = wp & 0xFFFFu;
              v[1] = wp >> 16;
            } else {
              v[0] = to16<false>(__uint_as_float(wp << 16));
              v[1] = to16<false>(__uint_as_float(wp & 0xFFFF0000u));
            }
          } else if constexpr (PAY == 2) {
            const uint32_t w32 = bf16_in_f32(e.x, raw_dword(rgp[0], u), u & 3);
            v[0] = OBF ? (w32 >> 16) : to16<false>(__uint_as_float(w32));
          } else {
            v[0] = to16<OBF>(exact_product((float)__builtin_bit_cast(_Float16, (uint16_t)(e.y >> 16)), scale));
          }
#pragma unroll
          for (int i = 0; i < KW; ++i) {
            const int wi = (u % FS) * KW + i;               // weight index in the segment
            if (wi & 1) pk[wi >> 1] |= v[i] << 16;
            else pk[wi >> 1] = v[i];
            // built here, not sunk to the flush with every step's table entry live
            asm volatile("" : "+v"(pk[wi >> 1]));
          }
          renorm_step<RAGGED>(x, rposb, ring, active);
          if ((u + 1) % FS == 0) {
            // segment of steps [j + u + 1 - FS, j + u]: stage, then store row-contiguous
            const uint32_t sb = stage + lane * kStagePitch;
#pragma unroll
            for (int c = 0; c < CPR; ++c)
              lds_store4(sb + 16 * c, make_uint4(pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]));
            __builtin_amdgcn_wave_barrier();
            const uint64_t c0 = colw + (uint64_t)(j + u + 1 - FS) * KW;
#pragma unroll
            for (int r = 0; r < CPR; ++r) {
              const uint32_t ci = (uint32_t)r * 64 + lane, rr = ci / CPR, part = ci % CPR;
              const uint4 val = lds_load4(stage + rr * kStagePitch + part * 16);
              const uint32_t orow = rg * 64 + rr;
              if (!RAGGED || orow < a.rows)
                __builtin_nontemporal_store(ecw_u32x4{val.x, val.y, val.z, val.w},
                                            reinterpret_cast<ecw_u32x4*>(out + (uint64_t)orow * a.cols + c0 + part * 8));
            }
            __builtin_amdgcn_wave_barrier();
          }
        }
      }
    }
    if constexpr (BF2 || QD) {
      // the escaped weights' zeros of this tile are in flight: let the stores land
      // before their corrections overwrite them (other lanes wrote them)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      float acc_unused[1] = {0.f};
      tile_corrections<1, OBF ? kOutBf16 : kOutF16, false, QD>(a, rposb, haveb, nc, pre, wl, src, nch, lane, ring,
                                                              0, 0, KW * S, active, (uint64_t)row * a.cols + colw,
                                                              acc_unused, scale);
    }
  }
}

// Two word streams per wave (fused GEMV only): the tiles of row groups rg and rg + 1
// at the same slices [sl0, sl1) are decoded in lockstep.  The two dependency chains
// (table read -> state update -> ballot / prefix -> ring read) interleave, and both
// streams multiply the same activation columns, so every activation read is shared.
// Both tiles of a slice have the same number of steps: the loop has no per-step
// branch.  Only stream B (the higher row group) can be ragged.  Each lane sums its
// own row in step order, exactly as a one-stream wave does, so the results are the
// same bits.  INT codes and FP8 only.
template <int PAY, int CB, int KW, int B, bool RAGGED, bool XBF>
__device__ __forceinline__ void wave_body_rows2(const TArgs& a, const StreamHead& hA, const StreamHead& hB,
                                                uint32_t lut, uint32_t xs, uint32_t ringA, uint32_t ringB,
                                                uint32_t rg, uint32_t sl0, uint32_t sl1, uint32_t c_lo,
                                                uint32_t lane, bool activeB, float* accA, float* accB) {
  static_assert(PAY == 1 || PAY == 3, "two row streams per wave: INT codes and FP8 only");
  constexpr int U = 16;
  constexpr bool QF = kQuadF<PAY, CB, KW, false, XBF>;   // INT quads (fp16 x): codes in the entries
  static_assert(!kQuad<PAY, CB, KW> || QF, "two streams of INT quads: fp16 activations only");
  constexpr bool DOT = kDot<PAY, KW>;
  constexpr bool CLEAN = kCleanBias<PAY, CB, KW>;
  constexpr int XW = DOT ? (KW / 2) * B : KW * B;
  const uint32_t m = a.log2m, mmask = (1u << m) - 1u;

  // ring B sits at a fixed distance after ring A: one lane address serves both
  const uint32_t wl = ringA + lane * 8;
  head_ring(hA, wl, lane);
  head_ring(hB, wl + 2 * kRingStride, lane);
  const uint32_t nchA = hA.nch, nchB = hB.nch;
  const uint2* srcA = hA.src;
  const uint2* srcB = hB.src;
  uint32_t rposA = hA.rposb, rposB = hB.rposb;
  uint2 preA = hA.pre, preB = hB.pre;
  uint32_t haveA = 4 * kChunk, ncA = 2, haveB = 4 * kChunk, ncB = 2;
  uint32_t stA = hA.st, stB = hB.st;
  const uint32_t tA0 = rg * a.n_sl, tB0 = tA0 + a.n_sl;

  for (uint32_t sl = sl0; sl < sl1; ++sl) {
    uint32_t xA = stA, xB = stB;
    if (sl + 1 < sl1) {
      stA = a.states[(uint64_t)(tA0 + sl + 1) * 64 + lane];
      stB = a.states[(uint64_t)(tB0 + sl + 1) * 64 + lane];
    }
    const uint32_t S = (sl + 1 == a.n_sl) ? a.s_last : a.s_full;
    const uint32_t col = sl * a.tile_cols - c_lo;
    for (uint32_t j = 0; j < S; j += U) {
      prio_by_work_left(S - j, S);
      const uint32_t xg = xs + ((col + KW * j) * B / (DOT ? 2 : 1)) * 4;
#pragma unroll
      for (int qtr = 0; qtr < U / 4; ++qtr) {
        refill(rposA, haveA, ncA, preA, wl, srcA, nchA, lane);
        refill(rposB, haveB, ncB, preB, wl + 2 * kRingStride, srcB, nchB, lane);
        uint4 xq[XW];
#pragma unroll
        for (int i = 0; i < XW; ++i) xq[i] = lds_load4(xg + (qtr * XW + i) * 16);
#pragma unroll
        for (int u4 = 0; u4 < 4; ++u4) {
          const uint32_t* xw = reinterpret_cast<const uint32_t*>(xq) + u4 * XW;
          if constexpr (QF) {
            // both streams' table reads, then both ring reads, with the codes'
            // products issued while the ring reads are in flight
            const uint2 eA = decode_step_q(xA, lut, m, mmask);
            const uint2 eB = decode_step_q(xB, lut, m, mmask);
            const RenormRead rA = renorm_read<false>(xA, rposA, ringA, true);
            const RenormRead rB = renorm_read<RAGGED>(xB, rposB, ringB, activeB);
            const uint32_t a01 = __builtin_amdgcn_perm(eA.y, eA.y, 0x010C000Cu);
            const uint32_t a23 = __builtin_amdgcn_perm(eA.y, eA.y, 0x030C020Cu);
            const uint32_t b01 = __builtin_amdgcn_perm(eB.y, eB.y, 0x010C000Cu);
            const uint32_t b23 = __builtin_amdgcn_perm(eB.y, eB.y, 0x030C020Cu);
#pragma unroll
            for (int b = 0; b < B; ++b) {
              accA[b] = dot2<false>(a01, xw[b], accA[b]);
              accA[b] = dot2<false>(a23, xw[B + b], accA[b]);
              accB[b] = dot2<false>(b01, xw[b], accB[b]);
              accB[b] = dot2<false>(b23, xw[B + b], accB[b]);
            }
            pin<B>(accA);
            pin<B>(accB);
            renorm_apply2(rA, xA, rposA, rB, xB, rposB);
          } else {
            const uint2 eA = decode_step<CLEAN>(xA, lut, m, mmask);
            const uint2 eB = decode_step<CLEAN>(xB, lut, m, mmask);
            mac<PAY, CB, KW, B, XBF>(eA, xw, 0u, 0, accA);
            mac<PAY, CB, KW, B, XBF>(eB, xw, 0u, 0, accB);
            pin<B>(accA);
            pin<B>(accB);
            const RenormRead rA = renorm_read<false>(xA, rposA, ringA, true);
            const RenormRead rB = renorm_read<RAGGED>(xB, rposB, ringB, activeB);
            renorm_apply2(rA, xA, rposA, rB, xB, rposB);
          }
        }
      }
    }
    if constexpr (QF) {
      // each stream's escaped codes, from its own correction stream
      const uint64_t rowA = (uint64_t)rg * 64 + lane;
      tile_corrections<B, kOutAcc, XBF, false, true>(a, rposA, haveA, ncA, preA, wl, srcA, nchA, lane, ringA, xs, col,
                                                     KW * S, true, rowA * a.cols + (uint64_t)sl * a.tile_cols, accA);
      tile_corrections<B, kOutAcc, XBF, false, true>(a, rposB, haveB, ncB, preB, wl + 2 * kRingStride, srcB, nchB,
                                                     lane, ringB, xs, col, KW * S, activeB,
                                                     (rowA + 64) * a.cols + (uint64_t)sl * a.tile_cols, accB);
    }
  }
}

// ---- E8 lattice fields (EntroPack page, Sections 3.2, 3.3 and A.3)
//
// Per block of 8 weights a lane decodes 9 symbols: the coset c (table 0), then
// z1..z7 and m = floor(z8 / 2) from table 1 + 8c + j.  The inverse of the parity
// reduction is z8 = 2m + ((z1 + .. + z7) mod 2); the doubled coordinates are
// 2v = 2z + c.  Reconstruction: INT8 route 2v (the row scale is halved in the
// epilogue), FP8 route e4m3_rne(v) from a 256-entry LDS table indexed by 2v.
// Table entries are staged compactly as 4 bytes: f (12 bits) | bias (11 bits) << 12 |
// field value (int8) << 24, which needs M <= 2^11.
constexpr uint32_t kE8F8TableBytes = 1024;   // 256 x u32, fp16 value in the high half

template <bool MAT>
__device__ __forceinline__ int e8_decode(uint32_t& x, uint32_t addr, uint32_t m) {
  const uint32_t e = *lds_ptr<const uint32_t>(addr);
  x = mad_u24(x >> m, e & 0xFFFu, (e >> 12) & 0x7FFu);
  return (int)e >> 24;
}

// Dequantising decode of lattice fields (DQ = 1: fp16, 2: bf16; decode-only): each
// weight is v * row scale (INT8 route: 2v / 2) or e4m3(v) * row scale (FP8 route),
// exact in fp32 and rounded once.  Segments of four blocks (32 weights, 64 B) are
// stored row-contiguous through the wave's LDS tile, a quarter of the rows at a time
// (16 rows x kStagePitch; the 17 tables leave little LDS); a tile whose last slice
// ends on a partial segment stores its remaining blocks' chunks only.
template <int DQ>
__device__ __forceinline__ void e8_store_segment(const TArgs& a, const uint32_t* pk, uint32_t nck, uint32_t stage,
                                                 uint32_t rg, uint64_t c0, uint32_t lane) {
  uint16_t* out = static_cast<uint16_t*>(a.deq_out);
  const uint32_t rr = lane >> 2, part = lane & 3;
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    if ((lane >> 4) == (uint32_t)qq) {
      const uint32_t sb = stage + (lane & 15) * kStagePitch;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if ((uint32_t)c < nck)
          lds_store4(sb + 16 * c, make_uint4(pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]));
    }
    __builtin_amdgcn_wave_barrier();
    const uint32_t orow = rg * 64 + (uint32_t)qq * 16 + rr;
    if (part < nck && orow < a.rows) {
      const uint4 val = lds_load4(stage + rr * kStagePitch + part * 16);
      __builtin_nontemporal_store(ecw_u32x4{val.x, val.y, val.z, val.w},
                                  reinterpret_cast<ecw_u32x4*>(out + (uint64_t)orow * a.cols + c0 + part * 8));
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int B, bool MAT, bool RAGGED, bool F8, int DQ = 0>
__device__ __forceinline__ void wave_body_e8(const TArgs& a, const StreamHead& h, uint32_t lut, uint32_t xs,
                                             uint32_t ring, uint32_t f8tab, uint32_t rg, uint32_t t0, uint32_t t1,
                                             uint32_t c_lo, uint32_t lane, bool active, float* acc,
                                             uint32_t stage = 0) {
  static_assert(DQ == 0 || MAT, "dequantising decode is decode-only");
  const uint32_t m = a.log2m, mmask = (1u << m) - 1u;
  const uint32_t tbytes = 4u << m;                 // bytes per compact table
  const uint32_t row = rg * 64 + lane;
  const uint32_t sl0 = rg * a.n_sl;

  const uint32_t wl = ring + lane * 8;
  head_ring(h, wl, lane);
  const uint32_t gb = h.gb, nch = h.nch;
  const uint2* src = h.src;
  uint32_t rposb = h.rposb;
  uint2 pre = h.pre;
  uint32_t haveb = 4 * kChunk, nc = 2;
  uint32_t st = h.st;
  float scale = 0.f;                      // dequantising decode: the row scale
  if constexpr (DQ != 0) scale = active ? (float)__builtin_bit_cast(_Float16, a.scales[row]) : 0.f;
  uint32_t pk[DQ != 0 ? 16 : 1];          // dequantising decode: 4 blocks as packed 16-bit values

  for (uint32_t t = t0; t < t1; ++t) {
    uint32_t x = st;
    if (t + 1 < t1) st = a.states[(uint64_t)(t + 1) * 64 + lane];
    const uint32_t sl = t - sl0;
    const uint32_t S = (sl + 1 == a.n_sl) ? a.s_last : a.s_full;
    const uint32_t col0 = sl * a.tile_cols - c_lo;
    const uint32_t nblk = S / 9;
    for (uint32_t blk = 0; blk < nblk; ++blk) {
      prio_by_work_left(nblk - blk, nblk);
      const uint32_t step0 = blk * 9;
      // activations of the block's 8 columns: fp32 [col][B]
      float xv[MAT ? 1 : 8 * B];
      if constexpr (!MAT) {
#pragma unroll
        for (int i = 0; i < 2 * B; ++i) {
          const uint4 q = lds_load4(xs + ((col0 + 8 * blk) * B) * 4 + i * 16);
          xv[4 * i] = __uint_as_float(q.x);
          xv[4 * i + 1] = __uint_as_float(q.y);
          xv[4 * i + 2] = __uint_as_float(q.z);
          xv[4 * i + 3] = __uint_as_float(q.w);
        }
      }
      refill(rposb, haveb, nc, pre, wl, src, nch, lane);
      const int c = e8_decode<MAT>(x, lut + ((x & mmask) << 2), m) & 1;    // coset, table 0
      if constexpr (MAT) {
        if ((!RAGGED || active) && a.sym_out) {
          const int32_t off0 = *reinterpret_cast<const int32_t*>(a.tables + 4);
          a.sym_out[(uint64_t)row * a.syms_per_row + (uint64_t)sl * a.s_full + step0] = (uint16_t)(c - off0);
        }
      }
      renorm_step<RAGGED>(x, rposb, ring, active);
      const uint32_t tb = lut + (1u + 8u * (uint32_t)c) * tbytes;          // table 1 + 8c
      int zsum = 0;
#pragma unroll
      for (int j = 1; j <= 8; ++j) {
        if (j == 4 || j == 8) refill(rposb, haveb, nc, pre, wl, src, nch, lane);
        const int v = e8_decode<MAT>(x, tb + (uint32_t)(j - 1) * tbytes + ((x & mmask) << 2), m);
        int z;
        if (j < 8) {
          z = v;
          zsum += v;
        } else {
          z = 2 * v + (zsum & 1);                                         // z8 from m and parity
        }
        const int w2 = 2 * z + c;                                         // doubled coordinate
        if constexpr (DQ != 0) {
          float val;
          if constexpr (F8) {
            const uint32_t hh = *lds_ptr<const uint32_t>(f8tab + ((uint32_t)(w2 + 128) & 255u) * 4) >> 16;
            val = exact_product((float)__builtin_bit_cast(_Float16, (uint16_t)hh), scale);
          } else {
            val = exact_product((float)w2 * 0.5f, scale);
          }
          const uint32_t v16 = to16<DQ == 2>(val);
          // weight j - 1 of block blk % 4 in the segment: word (blk % 4) * 4 + (j - 1) / 2
          // (blk is a runtime value: select the word among the four candidates)
          const uint32_t bq = blk & 3u;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int wi = w * 4 + (j - 1) / 2;
            if (bq == (uint32_t)w) {
              if ((j - 1) & 1) pk[wi] |= v16 << 16;
              else pk[wi] = v16;
            }
          }
        } else if constexpr (!MAT) {
          if constexpr (F8) {
            const uint32_t h = *lds_ptr<const uint32_t>(f8tab + ((uint32_t)(w2 + 128) & 255u) * 4);
#pragma unroll
            for (int b = 0; b < B; ++b) acc[b] = fma_mix_hi(h, xv[(j - 1) * B + b], acc[b]);
          } else {
            const float wf = (float)w2;
#pragma unroll
            for (int b = 0; b < B; ++b) acc[b] = fmaf(wf, xv[(j - 1) * B + b], acc[b]);
          }
        } else if (!RAGGED || active) {
          const uint32_t step = step0 + (uint32_t)j;
          if (a.sym_out) {
            const uint32_t tbl = 1u + 8u * (uint32_t)c + (uint32_t)(j - 1);
            const int32_t off = *reinterpret_cast<const int32_t*>(a.tables + (uint64_t)tbl * 520 + 4);
            a.sym_out[(uint64_t)row * a.syms_per_row + (uint64_t)sl * a.s_full + step] = (uint16_t)(v - off);
          }
          if (a.w_out) {
            const uint64_t wi = (uint64_t)row * a.cols + (uint64_t)col0 + c_lo + 8ull * blk + (uint64_t)(j - 1);
            if constexpr (F8)
              static_cast<uint8_t*>(a.w_out)[wi] =
                  (uint8_t)(*lds_ptr<const uint32_t>(f8tab + ((uint32_t)(w2 + 128) & 255u) * 4));
            else
              static_cast<int8_t*>(a.w_out)[wi] = (int8_t)w2;
          }
        }
        renorm_step<RAGGED>(x, rposb, ring, active);
      }
      if constexpr (DQ != 0) {
        if ((blk & 3u) == 3u)
          e8_store_segment<DQ>(a, pk, 4, stage, rg, (uint64_t)sl * a.tile_cols + 8ull * (blk - 3), lane);
      }
    }
    if constexpr (DQ != 0) {
      if (nblk & 3u)                      // the last slice's partial segment
        e8_store_segment<DQ>(a, pk, nblk & 3u, stage, rg, (uint64_t)sl * a.tile_cols + 8ull * (nblk & ~3u), lane);
    }
    if constexpr (MAT) {
      const bool ok_lane = !active || x == kStateL;
      const uint64_t bad = __ballot(!ok_lane);
      if (lane == 0 && a.status_out)
        a.status_out[t] = (bad != 0 ? 1u : 0u) | ((rposb != (a.offsets[t + 1] - gb) * 2) ? 2u : 0u);
    }
  }
}

// E4M3 byte nearest to t / 2 (t = 0..128), ties to the even code: t is rounded to a
// 4-bit significand (implicit one and 3 fraction bits) with round-half-even.
__device__ inline uint32_t e4m3_of_half_int(uint32_t t) {
  if (t == 0) return 0;
  int e2 = 31 - __builtin_clz(t);                  // t = 2^e2 * 1.f
  uint32_t q;
  if (e2 <= 3) {
    q = t << (3 - e2);                             // exact: 1.fff in 4 bits
  } else {
    const int sh = e2 - 3;
    q = t >> sh;
    const uint32_t rem = t & ((1u << sh) - 1), half = 1u << (sh - 1);
    if (rem > half || (rem == half && (q & 1u))) ++q;
    if (q == 16) {
      q = 8;
      ++e2;
    }
  }
  // value = q * 2^(e2 - 3) / 2 = (q / 8) * 2^(e2 - 1); biased exponent e2 - 1 + 7
  return ((uint32_t)(e2 + 6) << 3) | (q & 7u);
}

// fp16 bits of a normal E4M3 byte's value (the table only holds normal codes and 0)
__device__ inline uint32_t fp16_of_e4m3_normal(uint32_t b) {
  const uint32_t e = (b >> 3) & 0xF, mnt = b & 7, sign = (b & 0x80) << 8;
  if ((b & 0x7F) == 0) return sign;
  return sign | ((e - 7 + 15) << 10) | (mnt << 7);
}

// 16-bit float bits of a small integer, in the activations' type.
template <bool XBF>
__device__ __forceinline__ uint32_t small_int_bits(int q) {
  if constexpr (XBF) return __float_as_uint((float)q) >> 16;     // exact for |q| < 2^8
  else return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)q);
}

// PAY: 1 INT codes, 2 BF16 exponent, 3 FP8.  CB/KW: code bits and codes per symbol
// (INT).  B: batch capacity (1 or 4).  MAT: decode-only test hook.  XBF: the dot path
// multiplies bf16 activations (else fp16).
// Block = W waves on consecutive slices of one row group; wave w owns R consecutive
// tiles, decoded one after the other as one word stream or, for the fused GEMV of
// INT (one or two codes per symbol) and FP8 payloads with R >= 2, as two streams
// (first and second half) in lockstep.
// LDS, from address 0 (the kernel declares no static LDS): [pair side table]
// [decode table] [activations] [rings].
// Register budget: batch-1 kernels are held to 64 VGPRs so 8 waves fit per SIMD (two
// 16-wave blocks per CU) and hide the LDS latency of the decode chain.
template <int B>
constexpr int kWavesPerEU = B == 1 ? 8 : 4;
// Decode-only kernels of BF16 payloads (raw-byte groups and a 32-weight output
// segment beside the decode state) and the dequantising decode of lattice fields get
// 128 VGPRs instead of spilling.
template <int PAY, int B, bool MAT, bool XBF>
constexpr int kKernelWaves = (MAT && (PAY == 2 || (PAY == 4 && XBF))) ? 4 : kWavesPerEU<B>;

// Decode-only kernels (MAT) do not multiply activations, so XBF selects their output
// instead: false = the test hook's symbols / logical weights / tile status, true =
// the dequantising decode's dense matrix.
template <int PAY, int CB, int KW, int B, bool MAT, bool XBF>
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(kKernelWaves<PAY, B, MAT, XBF>)))
k_decode(const uint32_t n_blocks, const uint32_t nt, const uint32_t waves, const uint32_t grid,
         const uint32_t bb1, const uint32_t bb2, const uint32_t bb3, const uint32_t bb4, const uint32_t bb5,
         const uint32_t bb6, const uint32_t bb7, const KArgs ka) {
  extern __shared__ __align__(16) unsigned char smem[];
  (void)smem;
  __builtin_amdgcn_s_setprio(3);           // see prio_by_work_left
  // activations staged as packed 16-bit pairs (dot-product paths), else as fp32
  constexpr bool DOT = (kDot<PAY, KW> || kBfPair<PAY, KW, XBF> || (kBfSym2<PAY, KW> && XBF)) && !MAT;
  constexpr bool DEQ = MAT && XBF;
  constexpr bool QD = kQuad<PAY, CB, KW>;
  constexpr bool QF = kQuadF<PAY, CB, KW, MAT, XBF>;
  constexpr bool PTAB = kPairTable<PAY, KW, XBF> && !MAT && !QD;
  const uint32_t W = waves;
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wid = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Hardware block b runs on XCD b % 8.  Give each XCD a contiguous range of logical
  // blocks (the slice groups of one row group are adjacent).  The grid (`grid`) is
  // a multiple of 8; surplus blocks exit at once.
  const uint32_t per = grid >> 3;
  const uint32_t gl = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (gl >= n_blocks) return;
  // tensor of a grouped launch: blocks are numbered tensor by tensor
  static_assert(kMaxGroup == 8, "one preloaded argument per group member after the first");
  uint32_t ti = 0, bbt = 0;
  const uint32_t bbs[kMaxGroup] = {0u, bb1, bb2, bb3, bb4, bb5, bb6, bb7};
#pragma unroll
  for (uint32_t i = 1; i < kMaxGroup; ++i)
    if (i < nt && gl >= bbs[i]) { ti = i; bbt = bbs[i]; }
  const TArgs& a = ka.t[ti];
  const uint32_t lb = gl - bbt;
  constexpr bool E8 = PAY == 4;
  // streams per wave: 2 = the tiles of two adjacent row groups in lockstep (fused
  // GEMV of INT and FP8 payloads)
  constexpr bool kTwoCapable = !MAT && !E8 && PAY != 2 && (!QD || QF);
  const uint32_t NSr = (kTwoCapable && a.ns == 2) ? 2u : 1u;
  // the block's slice group and its run of row-group units [u_lo, u_hi); a unit is
  // NSr adjacent row groups, decoded by the waves' streams
  const uint32_t rgi = lb / a.n_sg, sg = lb - rgi * a.n_sg;
  const uint32_t n_units = (a.n_rg + NSr - 1) / NSr;
  const uint32_t u_lo = rgi * a.rpb, u_hi = min(u_lo + a.rpb, n_units);
  uint32_t rg = u_lo * NSr;
  const uint32_t R = a.tiles_per_wave;
  const uint32_t sl_blk = sg * W * R;
  const uint32_t sl_blk_end = min(sl_blk + W * R, a.n_sl);
  const uint32_t c_lo = sl_blk * a.tile_cols;
  const uint32_t c_hi = min(sl_blk_end * a.tile_cols, a.cols);
  constexpr bool E8F8 = E8 && CB == 1;            // E8: CB selects the FP8 reconstruction
  // INT quads: the fused product with fp16 activations and the dequantising decode
  // take the codes from the decode entries; the bf16 product and the decode-only
  // hook read a tuple-indexed table (entries turned back into symbol form below)
  constexpr bool QT = QD && !QF && !DEQ;
  const uint32_t pair_bytes = QT   ? (a.quad_t * 8 + 15) & ~15u
                              : QD ? 0
                                   : PTAB ? kPairTableBytes : (E8F8 ? kE8F8TableBytes : 0);
  const uint32_t lut = pair_bytes;
  const uint32_t lut_bytes = a.lut_entries * (E8 ? 4 : 8);
  const uint32_t xs = lut + lut_bytes;
  const uint32_t xs_bytes = MAT ? 0 : ((a.xs_cols * B * (DOT ? 2 : 4) + 15) & ~15u);
  const uint32_t rings = xs + xs_bytes;
  // wave-uniform LDS addresses, pinned to scalar registers (the compiler otherwise
  // may carry them in VGPRs and pay a vector add per ring read)
  const uint32_t ring = __builtin_amdgcn_readfirstlane(rings + wid * NSr * (2 * kRingStride));
  const uint32_t ringB = __builtin_amdgcn_readfirstlane(ring + 2 * kRingStride);

  // this wave's tiles; their offsets and start states are requested before the
  // staging loads so both latencies overlap
  const uint32_t w_sl0 = min(sl_blk + wid * R, sl_blk_end);
  const uint32_t w_sl1 = min(w_sl0 + R, sl_blk_end);
  uint32_t tb = rg * a.n_sl;
  StreamHead hA, hB;
  bool hasB = NSr == 2 && rg + 1 < a.n_rg;        // wave-uniform
  head_begin(a, tb + w_sl0, tb + w_sl1, lane, hA);
  if (kTwoCapable && hasB) head_begin(a, tb + a.n_sl + w_sl0, tb + a.n_sl + w_sl1, lane, hB);

  // ---- A2 / A3 prologue.  Every global load is issued before the first wait: the
  // first round of the decode table (up to 4 x 16 bytes per thread) and of the
  // activations (16 bytes per thread) go out together with the stream heads; the
  // first word chunks follow as soon as the tile offsets (scalar loads) arrive; the
  // LDS writes come last.  Larger tables / activation slices than one round take a
  // second pass.
  const uint32_t bd = W * 64;
  constexpr int KL = 4;
  const uint32_t nl16 = E8 ? 0 : a.lut_entries / 2;              // table, 16-byte units
  const uint4* lsrc = reinterpret_cast<const uint4*>(a.lut);
  uint4 lv[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i) {
    const uint32_t idx = tid + (uint32_t)i * bd;
    if (idx < nl16) lv[i] = lsrc[idx];
  }
  // INT quads in symbol form: the first round of stored tuples goes out with the
  // table, ahead of the word chunks, so the staging barrier does not wait for the
  // chunks
  constexpr int KT = QT ? 4 : 1;
  const uint16_t* tup = reinterpret_cast<const uint16_t*>(a.tables + sizeof(TableRecord));
  uint32_t tv[KT];
  if constexpr (QT) {
#pragma unroll
    for (int i = 0; i < KT; ++i) {
      const uint32_t idx = tid + (uint32_t)i * bd;
      tv[i] = idx < a.quad_t ? tup[idx] : 0u;
    }
  }
  // activations, 8 columns per unit (none for the materialising hook; nvec stays a
  // valid divisor there)
  const uint32_t nvec = MAT ? 1u : a.xs_cols / 8;
  const uint32_t nxv = MAT ? 0u : nvec * B;
  auto x_load = [&](uint32_t v) {
    const uint32_t b = v / nvec, c8 = v - b * nvec, col = c_lo + 8 * c8;
    uint4 raw = {0u, 0u, 0u, 0u};
    if (col < c_hi && b < a.nb)
      raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + (uint64_t)b * a.cols + col);
    return raw;
  };
  auto x_store = [&](uint32_t v, const uint4 raw) {
    const uint32_t b = v / nvec, c8 = v - b * nvec;
    const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
    if constexpr (DOT) {
      if constexpr (B == 1) {
        lds_store4(xs + c8 * 16, raw);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) *lds_ptr<uint32_t>(xs + ((4 * c8 + i) * B + b) * 4) = w4[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint16_t h = (uint16_t)(w4[i >> 1] >> (16 * (i & 1)));
        const float f = a.x_is_bf16 ? __uint_as_float((uint32_t)h << 16) : (float)__builtin_bit_cast(_Float16, h);
        *lds_ptr<float>(xs + ((8 * c8 + i) * B + b) * 4) = f;
      }
    }
  };
  uint4 xv0 = {0u, 0u, 0u, 0u};
  if constexpr (!MAT) {
    if (tid < nxv) xv0 = x_load(tid);
  }
  // first word chunks of the stream(s): in flight across the LDS writes and barrier
  head_chunks(a, lane, hA);
  if (kTwoCapable && hasB) head_chunks(a, lane, hB);

  if constexpr (E8) {
    // E8 tables are packed to 4-byte entries on the way.  The 17 tables take several
    // rounds of the block, so the entries go in batches of eight rounds: eight loads
    // in flight (indices clamped into the table), then the eight LDS writes.
    const uint2* src = a.lut;
    const uint32_t ne = a.lut_entries;
    for (uint32_t i0 = 0; i0 < ne; i0 += 8 * bd) {       // wave-uniform
      uint2 e[8];
#pragma unroll
      for (uint32_t k = 0; k < 8; ++k) {
        const uint32_t i = i0 + k * bd + tid;
        e[k] = src[i < ne ? i : ne - 1];
      }
#pragma unroll
      for (uint32_t k = 0; k < 8; ++k) {
        const uint32_t i = i0 + k * bd + tid;
        if (i < ne)
          *lds_ptr<uint32_t>(lut + i * 4) = (e[k].x & 0xFFFu) | ((e[k].y & 0x7FFu) << 12) | (e[k].x & 0xFF000000u);
      }
    }
    if constexpr (E8F8) {
      for (uint32_t i = tid; i < 256; i += bd) {
        const int w2 = (int)i - 128;                 // doubled coordinate
        const uint32_t mag = e4m3_of_half_int((uint32_t)(w2 < 0 ? -w2 : w2));
        const uint32_t b = mag | (w2 < 0 ? 0x80u : 0u);
        *lds_ptr<uint32_t>(i * 4) = b | (fp16_of_e4m3_normal(b) << 16);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const uint32_t idx = tid + (uint32_t)i * bd;
      if (idx < nl16) lds_store4(lut + idx * 16, lv[i]);
    }
    for (uint32_t idx = tid + KL * bd; idx < nl16; idx += bd) lds_store4(lut + idx * 16, lsrc[idx]);
  }
  if constexpr (!MAT) {
    if (tid < nxv) x_store(tid, xv0);
    for (uint32_t v = tid + bd; v < nxv; v += bd) x_store(v, x_load(v));
  }
  if constexpr (QT) {
    // stored tuple i -> its four codes as two packed bf16 numbers (decode-only
    // kernels: the tuple's digits), at byte 8 i
    auto t_store = [&](uint32_t i, uint32_t v) {
      uint2 e = make_uint2(v, 0u);
      if constexpr (!MAT) {
        e.x = small_int_bits<XBF>((int)(v & 15) - 8) | (small_int_bits<XBF>((int)((v >> 4) & 15) - 8) << 16);
        e.y = small_int_bits<XBF>((int)((v >> 8) & 15) - 8) | (small_int_bits<XBF>((int)(v >> 12) - 8) << 16);
      }
      lds_store2(i * 8, e);
    };
#pragma unroll
    for (int i = 0; i < KT; ++i) {
      const uint32_t idx = tid + (uint32_t)i * bd;
      if (idx < a.quad_t) t_store(idx, tv[i]);
    }
    for (uint32_t i = tid + KT * bd; i < a.quad_t; i += bd) t_store(i, tup[i]);
  }
  if constexpr (PTAB) {
    // symbol -> its codes as 16-bit floats, packed two per word (digits low first)
    // (blocks may have fewer than 256 threads)
    for (uint32_t sy = tid; sy < 256; sy += bd) {
      constexpr int half = 1 << (CB - 1);
      constexpr uint32_t dmask = (1u << CB) - 1;
      uint32_t w[KW / 2];
#pragma unroll
      for (int p = 0; p < KW / 2; ++p)
        w[p] = small_int_bits<XBF>((int)((sy >> (CB * 2 * p)) & dmask) - half) |
               (small_int_bits<XBF>((int)((sy >> (CB * (2 * p + 1))) & dmask) - half) << 16);
      if constexpr (KW == 2)
        *lds_ptr<uint32_t>(sy * 4) = w[0];
      else
        lds_store2(sy * 8, make_uint2(w[0], w[1]));
    }
  }
  __syncthreads();
  if constexpr (QT) {
    // INT quad entries {f | bias << 16, the codes' fp16 high bytes} -> {f, bias | 8 s << 16}
    // with s the slot's symbol: the symbols' runs of slots are in symbol order and
    // each starts at bias 0, so s + 1 is the number of run starts up to the slot.
    // Each thread takes a contiguous range of slots; a block-wide prefix sum of their
    // start counts (wave totals in the rings' space, free until the streams start)
    // gives each range its first s.
    constexpr uint32_t KS = 16;                  // slots read per round, all in flight
    constexpr uint32_t kNoStart = 1u << 16;      // stand-in past the range: bias 1, not a start
    const uint32_t per = (a.lut_entries + bd - 1) / bd;
    const uint32_t s0 = min(tid * per, a.lut_entries), s1 = min(s0 + per, a.lut_entries);
    uint32_t cnt = 0;
    for (uint32_t c = s0; c < s1; c += KS) {
      uint32_t lo[KS];
#pragma unroll
      for (uint32_t k = 0; k < KS; ++k) lo[k] = c + k < s1 ? *lds_ptr<const uint32_t>(lut + (c + k) * 8) : kNoStart;
#pragma unroll
      for (uint32_t k = 0; k < KS; ++k) cnt += (lo[k] >> 16) == 0u ? 1u : 0u;
    }
    uint32_t incl = cnt;                         // inclusive prefix over the wave's lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t v = (uint32_t)__shfl_up((int)incl, (unsigned)d, 64);
      if ((int)lane >= d) incl += v;
    }
    if (lane == 63) *lds_ptr<uint32_t>(rings + wid * 4) = incl;
    __syncthreads();
    uint32_t sym = incl - cnt - 1u;              // starts before s0, minus one
    for (uint32_t w = 0; w < wid; ++w) sym += *lds_ptr<const uint32_t>(rings + w * 4);
    for (uint32_t c = s0; c < s1; c += KS) {
      uint32_t lo[KS];
#pragma unroll
      for (uint32_t k = 0; k < KS; ++k) lo[k] = c + k < s1 ? *lds_ptr<const uint32_t>(lut + (c + k) * 8) : kNoStart;
#pragma unroll
      for (uint32_t k = 0; k < KS; ++k) {
        if (c + k < s1) {
          const uint32_t bias = lo[k] >> 16;
          sym += bias == 0u ? 1u : 0u;
          lds_store2(lut + (c + k) * 8, make_uint2(lo[k] & 0xFFFFu, bias | ((8u * sym) << 16)));
        }
      }
    }
    __syncthreads();
  }

  for (;;) {
  const uint32_t row = rg * 64 + lane;
  const bool active = row < a.rows;
  const bool ragged = (rg + 1) * 64 > a.rows;     // wave-uniform
  // the row scale of this thread's first output of the epilogue, requested now so the
  // epilogue does not wait for it
  float sc0 = 1.f;
  if constexpr (!MAT && PAY != 2) {
    if (tid < 64u * B * (hasB ? 2u : 1u)) {
      const uint32_t r0 = (rg + tid / (64u * B)) * 64 + (tid & 63);
      if (r0 < a.rows) sc0 = (float)__builtin_bit_cast(_Float16, a.scales[r0]);
    }
  }
  float acc[2][B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[0][b] = acc[1][b] = 0.f;
  if (w_sl0 < w_sl1) {
    if constexpr (E8 && DEQ) {
      // quarter-height LDS tile per wave after the rings (the 17 tables leave little LDS)
      const uint32_t stage = __builtin_amdgcn_readfirstlane(rings + W * (2 * kRingStride) + wid * 16 * kStagePitch);
      const uint32_t ta = tb + w_sl0, tz = tb + w_sl1;
      if (a.deq_bf16)
        wave_body_e8<B, MAT, true, E8F8, 2>(a, hA, lut, xs, ring, 0, rg, ta, tz, c_lo, lane, active, acc[0], stage);
      else
        wave_body_e8<B, MAT, true, E8F8, 1>(a, hA, lut, xs, ring, 0, rg, ta, tz, c_lo, lane, active, acc[0], stage);
    } else if constexpr (E8) {
      if (ragged)
        wave_body_e8<B, MAT, true, E8F8>(a, hA, lut, xs, ring, 0, rg, tb + w_sl0, tb + w_sl1, c_lo, lane, active,
                                         acc[0]);
      else
        wave_body_e8<B, MAT, false, E8F8>(a, hA, lut, xs, ring, 0, rg, tb + w_sl0, tb + w_sl1, c_lo, lane, active,
                                          acc[0]);
    } else if (kTwoCapable && hasB) {
      if constexpr (kTwoCapable) {
        const bool activeB = row + 64 < a.rows;
        if ((rg + 2) * 64 > a.rows)
          wave_body_rows2<PAY, CB, KW, B, true, XBF>(a, hA, hB, lut, xs, ring, ringB, rg, w_sl0, w_sl1, c_lo,
                                                     lane, activeB, acc[0], acc[1]);
        else
          wave_body_rows2<PAY, CB, KW, B, false, XBF>(a, hA, hB, lut, xs, ring, ringB, rg, w_sl0, w_sl1, c_lo,
                                                      lane, activeB, acc[0], acc[1]);
      }
    } else if (DEQ) {
      if constexpr (DEQ) {
        // dequantising decode: each wave's LDS tile follows the block's rings
        const uint32_t stage = __builtin_amdgcn_readfirstlane(rings + W * (2 * kRingStride) + wid * 64 * kStagePitch);
        const uint32_t ta = tb + w_sl0, tz = tb + w_sl1;
        if (a.deq_bf16) {
          if (ragged)
            wave_body_deq<PAY, CB, KW, true, true>(a, hA, lut, ring, stage, rg, ta, tz, lane, active);
          else
            wave_body_deq<PAY, CB, KW, false, true>(a, hA, lut, ring, stage, rg, ta, tz, lane, active);
        } else {
          if (ragged)
            wave_body_deq<PAY, CB, KW, true, false>(a, hA, lut, ring, stage, rg, ta, tz, lane, active);
          else
            wave_body_deq<PAY, CB, KW, false, false>(a, hA, lut, ring, stage, rg, ta, tz, lane, active);
        }
      }
    } else if constexpr (!DEQ) {
      if (ragged)
        wave_body<PAY, CB, KW, B, MAT, true, XBF>(a, hA, lut, xs, ring, rg, tb + w_sl0, tb + w_sl1, c_lo, lane,
                                                  active, acc[0]);
      else
        wave_body<PAY, CB, KW, B, MAT, false, XBF>(a, hA, lut, xs, ring, rg, tb + w_sl0, tb + w_sl1, c_lo, lane,
                                                   active, acc[0]);
    }
  }
  if constexpr (!MAT) {
    // ---- A8: epilogue.  Reuse each stream's ring as its reduction slot.
#pragma unroll
    for (int b = 0; b < B; ++b) {
      *lds_ptr<float>(ring + (b * 64 + lane) * 4) = acc[0][b];
      if (NSr == 2) *lds_ptr<float>(ringB + (b * 64 + lane) * 4) = acc[1][b];
    }
    __syncthreads();
    const uint32_t nrg = hasB ? 2u : 1u;
    const float unit_scale = (E8 && !E8F8) ? 0.5f : 1.f;     // INT8 route: weights are 2v
    for (uint32_t i = tid; i < 64u * B * nrg; i += W * 64) {
      const uint32_t s = i / (64u * B), bi = i - s * (64u * B);
      const uint32_t b = bi >> 6, l = bi & 63, rgs = rg + s, r = rgs * 64 + l;
      // the block's wave slots added in wave order; unrolled so that eight reads are
      // in flight at a time instead of one read per add (16 waves were 16 dependent
      // LDS round trips at the end of every block)
      float sum = 0.f;
#pragma unroll 8
      for (uint32_t w = 0; w < W; ++w)
        sum += *lds_ptr<const float>(rings + (w * NSr + s) * (2 * kRingStride) + (b * 64 + l) * 4);
      if (a.n_sg == 1) {
        if (r < a.rows && b < a.nb) {
          const float sc = (PAY == 2) ? 1.f : (i == tid ? sc0 : (float)__builtin_bit_cast(_Float16, a.scales[r])) * unit_scale;
          a.y[(uint64_t)b * a.rows + r] = sum * sc;
        }
      } else {
        // agent-scope stores: they reach the level every block's agent-scope loads
        // read, with no cache write-back of the whole L2
        __hip_atomic_store(reinterpret_cast<uint32_t*>(a.partials) + (((uint64_t)rgs * a.n_sg + sg) * B + b) * 64 + l,
                           __float_as_uint(sum), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (a.n_sg > 1) {
      // The row group spans several blocks.  Each thread waits until its partial
      // stores are complete, then one thread takes the unit's ticket; the block that
      // draws the last ticket adds every block's partials in block order and resets
      // the ticket for the next call.  Partials and tickets are only touched by
      // agent-scope atomic operations, so the completed stores are what the last
      // block reads.
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const uint32_t flag = rings;                // LDS word; the reduction slots are read
      if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(a.tickets + rg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *lds_ptr<uint32_t>(flag) = old + 1 == a.n_sg ? 1u : 0u;
      }
      __syncthreads();
      if (*lds_ptr<const uint32_t>(flag)) {
        for (uint32_t i = tid; i < 64u * B * nrg; i += W * 64) {
          const uint32_t s = i / (64u * B), bi = i - s * (64u * B);
          const uint32_t b = bi >> 6, l = bi & 63, rgs = rg + s, r = rgs * 64 + l;
          const uint32_t* p = reinterpret_cast<const uint32_t*>(a.partials) + ((uint64_t)rgs * a.n_sg * B + b) * 64 + l;
          float sum = 0.f;
          for (uint32_t g0 = 0; g0 < a.n_sg; g0 += 8) {
            // up to 8 loads in flight, summed in block order
            float v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
              v[k] = g0 + k < a.n_sg
                         ? __uint_as_float(__hip_atomic_load(p + (uint64_t)(g0 + k) * B * 64, __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT))
                         : 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k)
              if (g0 + k < a.n_sg) sum += v[k];
          }
          if (r < a.rows && b < a.nb) {
            const float sc = (PAY == 2) ? 1.f : (i == tid ? sc0 : (float)__builtin_bit_cast(_Float16, a.scales[r])) * unit_scale;
            a.y[(uint64_t)b * a.rows + r] = sum * sc;
          }
        }
        if (tid == 0) __hip_atomic_store(a.tickets + rg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  // next unit of the block: new stream heads; the barrier keeps the rings (which
  // held the reduction slots) untouched until every thread has read them
  rg += NSr;
  if (rg >= u_hi * NSr || rg >= a.n_rg) break;
  tb = rg * a.n_sl;
  hasB = NSr == 2 && rg + 1 < a.n_rg;
  head_begin(a, tb + w_sl0, tb + w_sl1, lane, hA);
  if (kTwoCapable && hasB) head_begin(a, tb + a.n_sl + w_sl0, tb + a.n_sl + w_sl1, lane, hB);
  head_chunks(a, lane, hA);
  if (kTwoCapable && hasB) head_chunks(a, lane, hB);
  __syncthreads();
  }
}

__global__ void k_fill_zero(float* y, uint64_t n) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = 0.f;
}

// ------------------------------------------------------------------ host launch
using KernelFn = void (*)(uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t,
                         uint32_t, uint32_t, const KArgs);

template <int B, bool MAT, bool XBF>
static KernelFn pick_kernel(const ecw_coding& c) {
  switch (c.payload) {
    case ECW_P_INT_CODES:
      switch (c.code_bits * 16 + c.weights_per_symbol) {
        case 4 * 16 + 1: return k_decode<1, 4, 1, B, MAT, MAT && XBF>;
        case 4 * 16 + 2: return k_decode<1, 4, 2, B, MAT, XBF>;
        case 3 * 16 + 1: return k_decode<1, 3, 1, B, MAT, MAT && XBF>;
        case 3 * 16 + 2: return k_decode<1, 3, 2, B, MAT, XBF>;
        case 2 * 16 + 1: return k_decode<1, 2, 1, B, MAT, MAT && XBF>;
        case 2 * 16 + 2: return k_decode<1, 2, 2, B, MAT, XBF>;
        case 2 * 16 + 4: return k_decode<1, 2, 4, B, MAT, XBF>;
        case 4 * 16 + 4: return k_decode<1, 4, 4, B, MAT, XBF>;
      }
      return nullptr;
    case ECW_P_BF16_EXP:
      return c.weights_per_symbol == 2 ? k_decode<2, 0, 2, B, MAT, XBF> : k_decode<2, 0, 1, B, MAT, XBF>;
    case ECW_P_FP8_E4M3: return k_decode<3, 0, 1, B, MAT, MAT && XBF>;
    case ECW_P_E8_LATTICE:
      return c.recon_dtype == ECW_DT_FP8_E4M3 ? k_decode<4, 1, 8, B, MAT, MAT && XBF>
                                              : k_decode<4, 0, 8, B, MAT, MAT && XBF>;
  }
  return nullptr;
}

static KernelFn pick_gemv_kernel(const ecw_coding& c, int B, bool xbf) {
  if (B == 1) return xbf ? pick_kernel<1, false, true>(c) : pick_kernel<1, false, false>(c);
  return xbf ? pick_kernel<4, false, true>(c) : pick_kernel<4, false, false>(c);
}

// activations staged as packed 16-bit pairs: INT with several codes per symbol, and
// BF16 weights with bf16 activations
static bool dot_path(const ecw_coding& c, bool xbf) {
  return (c.payload == ECW_P_INT_CODES && c.weights_per_symbol >= 2) || (c.payload == ECW_P_BF16_EXP && xbf);
}
static bool pair_table(const ecw_coding& c, bool xbf) {
  if (quad_coding(c.payload, c.code_bits, c.weights_per_symbol)) return false;
  return c.payload == ECW_P_INT_CODES && (c.weights_per_symbol == 4 || (c.weights_per_symbol == 2 && xbf));
}

// Two row-group streams per wave: asked for, and built for the payload (INT codes
// and FP8; E8 and BF16 decode one stream per wave: the BF16 raw bytes of two streams
// do not fit the 64-register budget beside the decode state, and exponent pairs and
// INT quads would need a correction pass per stream).
// Two row-group streams per wave: INT codes and FP8 (INT quads with fp16 activations).
static bool two_streams(const ecw_tensor* t, bool xbf) {
  const ecw_coding& c = t->coding;
  return t->streams_per_wave == 2 && c.payload != ECW_P_E8_LATTICE && c.payload != ECW_P_BF16_EXP &&
         !(quad_coding(c.payload, c.code_bits, c.weights_per_symbol) && xbf);
}

// Dynamic LDS of one block: pair side table, decode table, staged activations,
// word rings.  Mirrors the layout k_decode computes.
static uint64_t lds_bytes(const ecw_tensor* t, uint32_t W, uint32_t R, uint32_t xs_cols, int B, bool mat,
                          bool xbf) {
  const bool dot = !mat && dot_path(t->coding, xbf);
  const bool e8 = t->coding.payload == ECW_P_E8_LATTICE;
  uint64_t pair = (!mat && pair_table(t->coding, xbf)) ? kPairTableBytes : 0;
  if (e8 && t->coding.recon_dtype == ECW_DT_FP8_E4M3) pair = kE8F8TableBytes;
  const bool quads = quad_coding(t->coding.payload, t->coding.code_bits, t->coding.weights_per_symbol);
  const uint64_t tuples = (8ull * t->coding.stored_tuples + 15) / 16 * 16;
  // the fused product with fp16 activations (!mat, !xbf) and the dequantising decode
  // (mat, xbf) read the codes of INT quads from the decode entries
  const bool quad_codes_in_entries = quads && mat == xbf;
  if (quads) pair = quad_codes_in_entries ? 0 : tuples;
  const uint64_t lut = ((uint64_t)t->n_tables << t->coding.log2_m) * (e8 ? 4 : 8) / 8;
  const uint64_t xs = mat ? 0 : ((uint64_t)xs_cols * B * (dot ? 2 : 4) + 15) / 16 * 16;
  const bool two = !mat && two_streams(t, xbf);
  (void)R;
  // dequantising decode: a 64-row tile per wave (lattice fields: 16 rows)
  const uint64_t stage = mat ? (uint64_t)W * (e8 ? 16 : 64) * kStagePitch : 0;
  const uint64_t rings = (uint64_t)W * (two ? 2 : 1) * kRingStride * 2;
  return pair + lut * 8 + xs + rings + stage;
}

uint64_t launch_lds_bytes(const ecw_tensor* t, uint32_t W, uint32_t R, int B, bool mat, bool xbf) {
  const uint32_t xs_cols = mat ? 0 : W * R * t->coding.tile_cols;
  return lds_bytes(t, W, R, xs_cols, B > 1 ? 4 : 1, mat, xbf);
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
  a.tables = base + t->off_tables;
  a.quad_t = quad_coding(t->coding.payload, t->coding.code_bits, t->coding.weights_per_symbol)
                 ? t->coding.stored_tuples : 0;
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
  const uint32_t kw = t->coding.payload == ECW_P_BF16_EXP ? t->coding.weights_per_symbol : 1;   // raw bytes per step
  a.raw_full_bytes = (uint32_t)(raw_group_count(t->steps_full * kw) * 1024);
  a.raw_rg_bytes = t->n_slices ? (uint32_t)((t->n_slices - 1) * raw_group_count(t->steps_full * kw) * 1024 +
                                            raw_group_count(t->steps_last * kw) * 1024) : 0;
}

static ecw_status check_tensor(const ecw_tensor* t) {
  if (!t) return fail(ECW_E_INVALID_ARG, "tensor is NULL");
  ecw_status st = check_coding(&t->coding);
  if (st != ECW_OK) return st;
  if (!t->device_blob) return fail(ECW_E_INVALID_ARG, "tensor has no device blob");
  if (reinterpret_cast<uintptr_t>(t->device_blob) % 256) return fail(ECW_E_INVALID_ARG, "device blob misaligned");
  if (t->coding.payload == ECW_P_E8_LATTICE && t->coding.log2_m > 11)
    return fail(ECW_E_UNSUPPORTED, "E8 decode stages 4-byte table entries: M must be at most 2^11");
  if (t->waves_per_block < 1 || t->waves_per_block > 16 || t->tiles_per_wave < 1 || t->tiles_per_wave > 4096 ||
      t->streams_per_wave > 2 || t->row_groups_per_block > 65536)
    return fail(ECW_E_INVALID_ARG, "launch shape out of range");
  if (t->coding.payload != ECW_P_E8_LATTICE && (t->steps_full % 16 || t->steps_last % 16))
    return fail(ECW_E_UNSUPPORTED, "steps per tile must be a multiple of 16");
  return ECW_OK;
}

static uint64_t align256(uint64_t v) { return (v + 255) / 256 * 256; }

// Workspace layout of a group: each tensor whose row groups span several blocks
// gets its tickets and then its partials, in tensor order, 256-byte aligned.
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
    // one kernel serves the launch: its template follows payload, code width, codes
    // per symbol and (lattice fields) the reconstruction route
    if (c.payload != c0.payload || c.code_bits != c0.code_bits || c.weights_per_symbol != c0.weights_per_symbol ||
        c.recon_dtype != c0.recon_dtype || c.cols != c0.cols || ts[i]->waves_per_block != ts[0]->waves_per_block)
      return fail(ECW_E_INVALID_ARG, "grouped tensors must share payload, code width, codes per symbol, "
                                     "reconstruction, cols and waves per block");
    if (c.rows && (!ys[i] || reinterpret_cast<uintptr_t>(ys[i]) % 16))
      return fail(ECW_E_INVALID_ARG, "y must be a 16-byte aligned device pointer");
  }
  if (ts[0]->coding.cols && (!x || reinterpret_cast<uintptr_t>(x) % 16))
    return fail(ECW_E_INVALID_ARG, "x must be a 16-byte aligned device pointer");
  return ECW_OK;
}

// Blocks and dynamic LDS bytes per block of one member of a fused launch with W
// waves per block.
static void member_geometry(const ecw_tensor* t, uint32_t W, int B, bool xbf, uint32_t* n_blocks, uint64_t* lds) {
  const uint32_t ns = two_streams(t, xbf) ? 2u : 1u;
  const uint32_t units = (t->n_row_groups + ns - 1) / ns;
  const uint32_t rpb = std::max(1u, t->row_groups_per_block);
  *n_blocks = (units + rpb - 1) / rpb * slice_groups(t);
  *lds = lds_bytes(t, W, t->tiles_per_wave, W * t->tiles_per_wave * t->coding.tile_cols, B, false, xbf);
}

// Fused decode + GEMV of a group of tensors that read the same x: one launch.
// tickets[i] / partials[i]: tensor i's arrival tickets and partial sums (used only
// when its row groups span several blocks).  Arguments already checked.
static ecw_status launch_core(ecw_stream stream, const ecw_tensor* const* ts, int n, const void* x, int x_dtype,
                              float* const* ys, int batch, uint32_t* const* tickets, float* const* partials) {
  const int B = batch > 1 ? 4 : 1;
  const uint32_t W = ts[0]->waves_per_block;
  KArgs ka{};
  uint64_t lds = 0;
  uint32_t blocks = 0;
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
    a.ns = t->streams_per_wave;
    a.rpb = std::max(1u, t->row_groups_per_block);
    a.n_sg = slice_groups(t);
    uint64_t member_lds = 0;
    member_geometry(t, W, B, x_dtype == ECW_DT_BF16, &a.n_blocks, &member_lds);
    ka.block_begin[ka.nt] = blocks;
    a.xs_cols = W * t->tiles_per_wave * t->coding.tile_cols;
    blocks += a.n_blocks;
    lds = std::max(lds, member_lds);
    if (a.n_sg > 1) {
      a.tickets = tickets[i];
      a.partials = partials[i];
    }
    ++ka.nt;
  }
  if (ka.nt == 0) return ECW_OK;
  ka.n_blocks = blocks;
  ka.waves = W;
  KernelFn fn = pick_gemv_kernel(ts[0]->coding, B, x_dtype == ECW_DT_BF16);
  if (!fn) return fail(ECW_E_UNSUPPORTED, "no kernel for this payload / code width");
  if (lds > 160 * 1024) return fail(ECW_E_UNSUPPORTED, "launch shape needs more than 160 KiB of LDS");
  if (!lds_attribute_set(fn)) return fail(ECW_E_HIP, "hipFuncSetAttribute failed");
  const uint32_t grid = (blocks + 7) / 8 * 8;
  ka.grid = grid;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(W * 64), (size_t)lds, (hipStream_t)stream, ka.n_blocks, ka.nt, ka.waves,
                     ka.grid, ka.block_begin[1], ka.block_begin[2], ka.block_begin[3], ka.block_begin[4],
                     ka.block_begin[5], ka.block_begin[6], ka.block_begin[7], ka);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(ECW_E_HIP, std::string("launch failed: ") + hipGetErrorString(err));
  return ECW_OK;
}

// The same launch with a caller-provided workspace (group_workspace layout).
static ecw_status launch_group(ecw_stream stream, const ecw_tensor* const* ts, int n, const void* x,
                               int x_dtype, float* const* ys, int batch, void* workspace, size_t ws_bytes) {
  ecw_status st = check_group(ts, n, batch, x_dtype, x, ys);
  if (st != ECW_OK) return st;
  uint64_t woff[kMaxGroup];
  const uint64_t need = group_workspace(ts, n, batch, woff);
  if (need && (!workspace || ws_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256))
    return fail(ECW_E_INVALID_ARG, "workspace missing, too small or not 256-byte aligned");
  uint32_t* tickets[kMaxGroup] = {};
  float* partials[kMaxGroup] = {};
  for (int i = 0; i < n; ++i) {
    if (!workspace_bytes(ts[i], batch)) continue;
    // tickets first: for one tensor they sit at the same place for every launch shape
    uint8_t* base = static_cast<uint8_t*>(workspace) + woff[i];
    tickets[i] = reinterpret_cast<uint32_t*>(base);
    partials[i] = reinterpret_cast<float*>(base + ticket_bytes(ts[i]));
  }
  return launch_core(stream, ts, n, x, x_dtype, ys, batch, tickets, partials);
}

// ---- allocation-free variant of dec_gemv.  Its workspace is a file-scope device
// array, one copy per GPU the library runs on, held until the process ends.  The
// arrival tickets sit in a fixed region at its start (so they are back at zero
// after every completed call, whatever the launch shape), the partial sums after
// them.  Host code never uses the array's name as an address: the per-device
// address comes from hipGetSymbolAddress, taken once per device.
constexpr uint64_t kScratchBytes = ECW_NOALLOC_TICKET_BYTES + ECW_NOALLOC_PARTIAL_BYTES;   // per device
constexpr uint64_t kScratchTicketBytes = ECW_NOALLOC_TICKET_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// This device's copy of `scratch`, set up on first use: its address, and its
// ticket region cleared by a fill kernel on `stream` (a kernel, not a memset, so
// a call under graph capture stays capturable).
static ecw_status scratch_for_device(ecw_stream stream, uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return fail(ECW_E_HIP, "hipGetDevice failed or device index out of range");
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return fail(ECW_E_HIP, "hipGetSymbolAddress(scratch) failed");
    }
    const uint64_t words = kScratchTicketBytes / 4;
    hipLaunchKernelGGL(k_fill_zero, dim3((uint32_t)((words + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                       static_cast<float*>(ptr), words);
    if (hipGetLastError() != hipSuccess) return fail(ECW_E_HIP, "scratch clear launch failed");
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<uint8_t*>(g_scratch_ptr[dev]);
  return ECW_OK;
}

static ecw_status launch_noalloc(ecw_stream stream, const ecw_tensor* t, const void* x, int x_dtype, float* y,
                                 int batch) {
  ecw_status st = check_group(&t, 1, batch, x_dtype, x, &y);
  if (st != ECW_OK) return st;
  uint32_t* tickets[1] = {nullptr};
  float* partials[1] = {nullptr};
  const uint64_t pb = partial_bytes(t, batch);
  if (pb) {
    if (ticket_bytes(t) > kScratchTicketBytes || pb > kScratchBytes - kScratchTicketBytes)
      return fail(ECW_E_UNSUPPORTED,
                  "launch needs " + std::to_string(ticket_bytes(t)) + " bytes of tickets and " + std::to_string(pb) +
                      " bytes of partial sums; the allocation-free entry point holds at most " +
                      std::to_string(kScratchTicketBytes) + " and " + std::to_string(kScratchBytes - kScratchTicketBytes));
    uint8_t* base = nullptr;
    st = scratch_for_device(stream, &base);
    if (st != ECW_OK) return st;
    tickets[0] = reinterpret_cast<uint32_t*>(base);
    partials[0] = reinterpret_cast<float*>(base + kScratchTicketBytes);
  }
  return launch_core(stream, &t, 1, x, x_dtype, &y, batch, tickets, partials);
}

}  // namespace ecw

using namespace ecw;

extern "C" ecw_status dec_gemv(ecw_stream stream, const ecw_tensor* t, const void* x, int x_dtype,
                               float* y, int batch, void* workspace, size_t ws_bytes) {
  clear_error();
  return launch_group(stream, &t, 1, x, x_dtype, &y, batch, workspace, ws_bytes);
}

extern "C" ecw_status dec_gemv_noalloc(ecw_stream stream, const ecw_tensor* t, const void* x, int x_dtype,
                                       float* y, int batch) {
  clear_error();
  return launch_noalloc(stream, t, x, x_dtype, y, batch);
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

extern "C" ecw_status dec_gemv_group_geometry(const ecw_tensor* const* t, int n, int batch, int x_dtype,
                                              uint32_t* grid_threads, uint32_t* block_threads, size_t* lds_bytes_out) {
  clear_error();
  if (!t || n < 1 || n > kMaxGroup || !grid_threads || !block_threads || !lds_bytes_out)
    return fail(ECW_E_INVALID_ARG, "bad arguments");
  if (batch < 1 || batch > 4) return fail(ECW_E_INVALID_ARG, "batch must be 1..4");
  if (x_dtype != ECW_DT_F16 && x_dtype != ECW_DT_BF16) return fail(ECW_E_INVALID_ARG, "x dtype must be F16 or BF16");
  for (int i = 0; i < n; ++i) {
    if (!t[i] || t[i]->waves_per_block < 1 || t[i]->waves_per_block > 16 || t[i]->tiles_per_wave < 1)
      return fail(ECW_E_INVALID_ARG, "bad tensor or launch shape");
    if (t[i]->waves_per_block != t[0]->waves_per_block)
      return fail(ECW_E_INVALID_ARG, "grouped tensors must share waves per block");
  }
  const uint32_t W = t[0]->waves_per_block;
  uint32_t blocks = 0;
  uint64_t lds = 0;
  for (int i = 0; i < n; ++i) {
    if (t[i]->coding.rows == 0 || t[i]->n_tiles == 0) continue;
    uint32_t nb = 0;
    uint64_t l = 0;
    member_geometry(t[i], W, batch > 1 ? 4 : 1, x_dtype == ECW_DT_BF16, &nb, &l);
    blocks += nb;
    lds = std::max(lds, l);
  }
  *grid_threads = (blocks + 7) / 8 * 8 * W * 64;
  *block_threads = W * 64;
  *lds_bytes_out = (size_t)lds;
  return ECW_OK;
}

extern "C" ecw_status dec_gemv_group(ecw_stream stream, const ecw_tensor* const* t, int n, const void* x,
                                     int x_dtype, float* const* y, int batch, void* workspace,
                                     size_t ws_bytes) {
  clear_error();
  return launch_group(stream, t, n, x, x_dtype, y, batch, workspace, ws_bytes);
}

// Mean microseconds per call of `reps` grouped launches captured as one graph (so
// host launch cost is not measured); one warm-up replay first.
static ecw_status time_group(ecw_stream stream, const ecw_tensor* const* ts, int n, const void* x, int x_dtype,
                             float* const* ys, int batch, void* ws, size_t ws_bytes, int reps, float* us) {
  hipStream_t s = (hipStream_t)stream;
  // a direct call first: reports an unlaunchable group with its own status
  ecw_status st = launch_group(stream, ts, n, x, x_dtype, ys, batch, ws, ws_bytes);
  if (st != ECW_OK) return st;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return fail(ECW_E_HIP, "hipEventCreate failed");
  }
  hipGraph_t g = nullptr;
  hipGraphExec_t ge = nullptr;
  bool ok = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) == hipSuccess;
  bool launched = ok;
  for (int r = 0; launched && r < reps; ++r)
    launched = launch_group(stream, ts, n, x, x_dtype, ys, batch, ws, ws_bytes) == ECW_OK;
  if (ok) ok = hipStreamEndCapture(s, &g) == hipSuccess && launched;
  float ms = 0.f;
  ok = ok && hipGraphInstantiate(&ge, g, nullptr, nullptr, 0) == hipSuccess;
  ok = ok && hipGraphLaunch(ge, s) == hipSuccess;
  ok = ok && hipEventRecord(e0, s) == hipSuccess;
  ok = ok && hipGraphLaunch(ge, s) == hipSuccess;
  ok = ok && hipEventRecord(e1, s) == hipSuccess;
  ok = ok && hipEventSynchronize(e1) == hipSuccess;
  ok = ok && hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
  if (ge) (void)hipGraphExecDestroy(ge);
  if (g) (void)hipGraphDestroy(g);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (!ok) return fail(ECW_E_HIP, "timing a captured launch failed");
  *us = ms * 1000.f / (float)reps;
  return ECW_OK;
}

extern "C" ecw_status dec_time_group(ecw_stream stream, const ecw_tensor* const* t, int n, const void* x,
                                     int x_dtype, float* const* y, int batch, void* workspace, size_t ws_bytes,
                                     int reps, float* us_out) {
  clear_error();
  if (!us_out || reps < 1 || reps > 1000) return fail(ECW_E_INVALID_ARG, "bad timing arguments");
  if (!stream) return fail(ECW_E_INVALID_ARG, "timing captures a graph: pass a created stream, not the default one");
  return time_group(stream, t, n, x, x_dtype, y, batch, workspace, ws_bytes, reps, us_out);
}

// Times each candidate launch shape of one tensor and keeps the fastest.
extern "C" ecw_status dec_tune_launch(ecw_stream stream, ecw_tensor* t, const void* x, int x_dtype, float* y,
                                      int batch, void* workspace, size_t ws_bytes, const uint32_t* shapes,
                                      int n_shapes, int reps, float* us_out) {
  clear_error();
  if (!t || !shapes || !us_out || n_shapes < 1 || reps < 1 || reps > 1000)
    return fail(ECW_E_INVALID_ARG, "bad tuning arguments");
  if (!stream) return fail(ECW_E_INVALID_ARG, "tuning captures a graph: pass a created stream, not the default one");
  const uint32_t W0 = t->waves_per_block, R0 = t->tiles_per_wave, S0 = t->streams_per_wave,
                 P0 = t->row_groups_per_block;
  float best = -1.f;
  uint32_t bestW = W0, bestR = R0, bestS = S0, bestP = P0;
  ecw_status result = ECW_OK;
  for (int i = 0; i < n_shapes; ++i) {
    us_out[i] = -1.f;
    t->waves_per_block = shapes[4 * i];
    t->tiles_per_wave = shapes[4 * i + 1];
    t->streams_per_wave = shapes[4 * i + 2];
    t->row_groups_per_block = shapes[4 * i + 3];
    float us = 0.f;
    const ecw_status st = time_group(stream, &t, 1, x, x_dtype, &y, batch, workspace, ws_bytes, reps, &us);
    if (st == ECW_E_HIP) {
      result = st;
      break;
    }
    if (st != ECW_OK) continue;                 // shape not launchable: skipped
    us_out[i] = us;
    if (best < 0.f || us < best) {
      best = us;
      bestW = t->waves_per_block;
      bestR = t->tiles_per_wave;
      bestS = t->streams_per_wave;
      bestP = t->row_groups_per_block;
    }
  }
  t->waves_per_block = bestW;
  t->tiles_per_wave = bestR;
  t->streams_per_wave = bestS;
  t->row_groups_per_block = bestP;
  if (result != ECW_OK) return result;
  if (best < 0.f) return fail(ECW_E_INVALID_ARG, "no launchable candidate shape");
  clear_error();
  return ECW_OK;
}

static ecw_status launch_decode_only(ecw_stream stream, const ecw_tensor* t, uint16_t* symbols, void* w_out,
                                     uint32_t* tile_status, void* deq_out, bool deq_bf16) {
  KArgs ka{};
  TArgs& a = ka.t[0];
  fill_tensor(t, a);
  a.sym_out = symbols;
  a.w_out = w_out;
  a.status_out = tile_status;
  a.deq_out = deq_out;
  a.deq_bf16 = deq_bf16 ? 1u : 0u;
  a.nb = 1;
  a.tiles_per_wave = 1;   // every tile restarts its stream: per-tile status is exact
  a.ns = 1;
  a.rpb = 1;
  const uint32_t W = std::min<uint32_t>(8, t->n_slices);
  a.n_sg = (t->n_slices + W - 1) / W;
  a.n_blocks = a.n_rg * a.n_sg;
  a.xs_cols = 0;
  ka.nt = 1;
  ka.n_blocks = a.n_blocks;
  ka.waves = W;
  ka.block_begin[0] = 0;
  KernelFn fn = deq_out ? pick_kernel<1, true, true>(t->coding) : pick_kernel<1, true, false>(t->coding);
  if (!fn) return fail(ECW_E_UNSUPPORTED, "no kernel for this payload / code width");
  const uint64_t lds = lds_bytes(t, W, 1, 0, 1, true, deq_out != nullptr);
  if (lds > 160 * 1024) return fail(ECW_E_UNSUPPORTED, "decode table needs more than 160 KiB of LDS");
  if (!lds_attribute_set(fn)) return fail(ECW_E_HIP, "hipFuncSetAttribute failed");
  const uint32_t grid = (ka.n_blocks + 7) / 8 * 8;
  ka.grid = grid;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(W * 64), (size_t)lds, (hipStream_t)stream, ka.n_blocks, ka.nt, ka.waves,
                     ka.grid, ka.block_begin[1], ka.block_begin[2], ka.block_begin[3], ka.block_begin[4],
                     ka.block_begin[5], ka.block_begin[6], ka.block_begin[7], ka);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(ECW_E_HIP, std::string("launch failed: ") + hipGetErrorString(err));
  return ECW_OK;
}

extern "C" ecw_status dec_materialize(ecw_stream stream, const ecw_tensor* t, uint16_t* symbols,
                                      void* w_out, uint32_t* tile_status) {
  clear_error();
  ecw_status st = check_tensor(t);
  if (st != ECW_OK) return st;
  if (t->n_tiles == 0) return ECW_OK;
  return launch_decode_only(stream, t, symbols, w_out, tile_status, nullptr, false);
}

extern "C" ecw_status dec_dequantize(ecw_stream stream, const ecw_tensor* t, void* w_out, int out_dtype) {
  clear_error();
  ecw_status st = check_tensor(t);
  if (st != ECW_OK) return st;
  if (out_dtype != ECW_DT_F16 && out_dtype != ECW_DT_BF16)
    return fail(ECW_E_INVALID_ARG, "output dtype must be F16 or BF16");
  if (t->coding.cols % 8) return fail(ECW_E_UNSUPPORTED, "cols must be a multiple of 8");
  if (t->coding.rows && t->coding.cols && (!w_out || reinterpret_cast<uintptr_t>(w_out) % 16))
    return fail(ECW_E_INVALID_ARG, "w_out must be a 16-byte aligned device pointer");
  if (t->n_tiles == 0) return ECW_OK;
  return launch_decode_only(stream, t, nullptr, nullptr, nullptr, w_out, out_dtype == ECW_DT_BF16);
}
