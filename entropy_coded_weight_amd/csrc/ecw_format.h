// Blob format version 2: layout shared by the host encoder, the validator and the
// device kernels of this library.  All integers little-endian.
//
//   [0, 256)        BlobHeader
//   sections, each starting on a 256-byte boundary, in this order:
//   TABLES   n_tables x TableRecord                        (alphabet, offset, freq)
//            BF16 pairs: then 16 bytes, the exponent of each digit
//            INT quads: the record's alphabet is n, the number of stored tuples,
//            and its freq is zero; then stored_tuples u16 tuples (the first n
//            ascending, the rest 0) and stored_tuples u16 frequencies (likewise)
//   LUT      n_tables x M x 8 B decode entries             (derived from freq)
//   STATES   n_tiles x 64 x u32 decoder start states       (inactive lanes: 2^16)
//   OFFSETS  (n_tiles + 1) x u32 word offsets into WORDS   (last = total words)
//   WORDS    u16 payload words of all tiles in tile order, then >= kWordPad bytes of
//            zero padding (the decoder's chunked loads may read past a tile's end)
//   RAW      BF16 only: per tile G = ceil(weights per row slice / 16) groups of
//            [64 lanes][16 bytes] (byte i of a lane's group g: column 16 g + i)
//   SCALES   rows x fp16 row scales (absent for BF16)
//
// Tile t = row_group * n_slices + slice covers rows [64 g, 64 g + 64) and the
// symbols of columns [slice * tile_cols, ...).  Inside a tile, words are in decoder
// order: step-major, lanes ascending (EntroPack page, Sections 3.6 and C.3: one
// wave per independent tile, 32-bit states, 16-bit words).
//
// BF16 pairs (k = 2): a symbol is two exponent digits d0 | d1 << 4 (even column
// low) into the 16 stored exponents; digit 0 is exponent 0.  A weight whose
// exponent is not stored is coded as digit 0 with raw byte 0 (+0.0) and escaped:
// after the tile's last ANS word comes its correction stream (MINE page, Section
// 4.1 "Escapes"): a 64-bit lane mask (4 words, low first; bit l = lane l has
// records), then records in rounds (round r: the r-th record of each lane with more
// than r, lanes ascending), each record two words, low half first:
//   bits 0..15 bf16 weight, 16..26 column in the slice, 27 last of its row, 28..31 0
//
// INT quads (4-bit codes, k = 4): a symbol is the index of a stored 4-tuple of codes
// (digit q + 8 of column 4j + i at bits 4i..4i+3); a tuple outside the table is
// coded as the stored tuple reached by setting the fewest of its codes to 0, and
// each nonzero code so set is escaped into the same correction stream, its record
// holding the code as a bf16 number.
//
// Decode entry of slot i (table t), symbol s, as two u32 (MINE page, Section 4.1:
// one table read yields both the state-update operands and the payload), every
// coding but INT quads:
//   lo = f | a8 << 24     f <= 2^13 sits in the low 24 bits, so the 24-bit multiply
//                         f * (x >> m) ignores a8
//   hi = bias | h16 << 16 bias = i - cum[s] < 2^13; next state = f * (x >> m) + bias
// a8 / h16 per payload (h16 is an fp16 bit pattern, exact for every value here):
//   INT, k = 1:       a8 = the code q0 (int8), h16 = fp16(q0)
//   INT, k = 2:       a8 = symbol (packed unsigned digits, first code lowest),
//                     h16 = hi8(fp16(q0)) | hi8(fp16(q1)) << 8 (the fp16 of a code
//                     |q| <= 8 has a zero low byte, so the two high bytes are the
//                     whole values)
//   INT, k = 4:       a8 = symbol, h16 = 0
//   BF16:             a8 = exponent byte rotated right by one bit (bit 0 in bit 7),
//                     h16 = 0.  With the raw byte (sign << 7 | mantissa) the bf16
//                     value's high byte is then sign | a8[6:0] and its low byte
//                     a8[7] | mantissa: whole bytes, joined with byte permutes
//   BF16, k = 2:      a8 = symbol, h16 = rot(e0) | rot(e1) << 8 with e0, e1 the
//                     digits' exponents and rot the rotation above
//   FP8 E4M3:         a8 = code byte, h16 = fp16(e4m3 value) (NaN codes: 0x7E00)
//   E8:               a8 = field value (int8), h16 = 0
// INT quads, with q0..q3 the four codes of the symbol's stored tuple:
//   lo = f | bias << 16   (f <= 2^13, bias < 2^13: two clean 16-bit halves)
//   hi = hi8(fp16(q0)) | hi8(fp16(q1)) << 8 | hi8(fp16(q2)) << 16 | hi8(fp16(q3)) << 24
// so the fused product with fp16 activations takes the state update and all four
// codes from one read; the other decoders recover the symbol index from the slot
// order (a slot with bias 0 starts the next symbol's run).
#pragma once
#include <stdint.h>

namespace ecw {

constexpr uint32_t kMagic = 0x31574345u;   // "ECW1"
constexpr uint32_t kVersion = 2;
constexpr uint32_t kHeaderBytes = 256;
constexpr uint32_t kLanes = 64;
constexpr uint32_t kStateL = 1u << 16;     // rANS lower bound L
constexpr uint32_t kSectionAlign = 256;
constexpr uint32_t kWordPad = 4096;        // zero bytes after the last word
constexpr uint32_t kMinLog2M = 8;
constexpr uint32_t kMaxLog2M = 13;
constexpr uint32_t kPairDigits = 16;        // BF16 pairs: stored exponents
constexpr uint32_t kEscLast = 1u << 27;     // correction record: last of its row
constexpr uint32_t kEscMaskWords = 4;       // correction stream: lane mask words
constexpr uint32_t kMaxTuples = 4096;       // INT quads: stored tuples at most
constexpr uint32_t kQuadZero = 0x8888;      // INT quads: the tuple of four zero codes

// INT quads: four 4-bit codes per symbol over a table of stored tuples
inline bool quad_coding(uint32_t payload, uint32_t code_bits, uint32_t k) {
  return payload == 1 && code_bits == 4 && k == 4;
}

enum Section : uint32_t {
  kSecTables = 0, kSecLut, kSecStates, kSecOffsets, kSecWords, kSecRaw, kSecScales, kNumSections
};

struct SectionRef {
  uint64_t offset;
  uint64_t bytes;
};

struct BlobHeader {
  uint32_t magic;
  uint32_t version;
  uint32_t header_bytes;
  uint32_t n_sections;
  // coding
  uint32_t payload, rows, cols, weights_per_symbol, code_bits, log2_m, tile_rows, tile_cols,
      recon_dtype;
  // derived geometry
  uint32_t n_tables, n_row_groups, n_slices, n_tiles, steps_full, steps_last, lut_entry_bytes;
  uint32_t stored_tuples;   // INT quads (else 0)
  uint32_t reserved1;
  uint64_t total_bytes;  // byte offset 88
  SectionRef sec[8];
  uint8_t pad[256 - 4 * 4 - 9 * 4 - 9 * 4 - 8 - 8 * 16];  // sections at byte offset 96
};
static_assert(sizeof(BlobHeader) == 256, "header must be 256 bytes");

struct TableRecord {          // 520 bytes
  uint32_t alphabet;
  int32_t value_offset;
  uint16_t freq[256];
};
static_assert(sizeof(TableRecord) == 520, "table record size");

inline uint32_t symbols_per_row_slice(uint32_t payload, uint32_t k, uint32_t tile_cols) {
  if (payload == 1 || payload == 2) return tile_cols / k;
  if (payload == 4) return tile_cols / 8 * 9;
  return tile_cols;
}
inline uint32_t symbols_per_row(uint32_t payload, uint32_t k, uint32_t cols) {
  if (payload == 1 || payload == 2) return cols / k;
  if (payload == 4) return cols / 8 * 9;
  return cols;
}
// BF16 raw plane: 16-byte groups per lane for `weights` columns of a tile
inline uint64_t raw_group_count(uint32_t weights) { return (weights + 15) / 16; }
inline uint32_t rot_exponent(uint32_t e) { return ((e >> 1) | (e << 7)) & 0xFF; }

// fp16 bit pattern of a small integer |v| <= 2048 (exact).
inline uint16_t fp16_of_int(int v) {
  if (v == 0) return 0;
  uint16_t sign = v < 0 ? 0x8000 : 0;
  uint32_t a = (uint32_t)(v < 0 ? -v : v);
  int e = 31 - __builtin_clz(a);                 // a = 2^e * 1.m
  uint32_t mant = (a << (10 - e)) & 0x3FF;
  return (uint16_t)(sign | ((uint32_t)(e + 15) << 10) | mant);
}

// fp16 bit pattern of an OCP E4M3 byte's value (every finite E4M3 value is an fp16
// value: 3 mantissa bits, exponents 2^-9 .. 2^8).
inline uint16_t fp16_of_e4m3(uint8_t b) {
  const uint16_t sign = (b & 0x80) ? 0x8000 : 0;
  const uint32_t e = (b >> 3) & 0xF, m = b & 7;
  if (e == 15 && m == 7) return 0x7E00;                       // NaN
  if (e == 0) {
    if (m == 0) return sign;                                  // +-0
    // m * 2^-9 = 1.f * 2^k with k = msb(m) - 9
    int k = 31 - __builtin_clz(m);
    uint32_t mant = (m << (10 - k)) & 0x3FF;
    return (uint16_t)(sign | ((uint32_t)(k - 9 + 15) << 10) | mant);
  }
  return (uint16_t)(sign | ((e - 7 + 15) << 10) | (m << 7));
}

// Decode entry of an INT quads slot: frequency f and bias of its symbol, whose stored
// tuple holds digit q + 8 of code i at bits 4i..4i+3 (see the layout above).
inline void quad_entry(uint32_t f, uint32_t bias, uint32_t tuple, uint32_t* lo, uint32_t* hi) {
  *lo = f | (bias << 16);
  uint32_t h = 0;
  for (int i = 0; i < 4; ++i)
    h |= (uint32_t)(fp16_of_int((int)((tuple >> (4 * i)) & 15) - 8) >> 8) << (8 * i);
  *hi = h;
}

// Table entry payload of symbol s (see the layout above).  pair_values: the BF16 pair
// stored exponents (else unused).
inline void entry_payload(uint32_t payload, uint32_t code_bits, uint32_t k, int32_t value_offset,
                          const uint8_t* pair_values, uint32_t s, uint32_t* a8, uint32_t* h16) {
  switch (payload) {
    case 1: {
      const int half = 1 << (code_bits - 1);
      const uint32_t mask = (1u << code_bits) - 1;
      if (k == 4) {
        *a8 = s & 0xFF;
        *h16 = 0;
      } else if (k == 2) {
        const int q0 = (int)(s & mask) - half;
        const int q1 = (int)((s >> code_bits) & mask) - half;
        *a8 = s & 0xFF;
        *h16 = (uint32_t)(fp16_of_int(q0) >> 8) | (uint32_t)(fp16_of_int(q1) & 0xFF00u);
      } else {
        const int q0 = (int)(s & mask) - half;
        *a8 = (uint32_t)(q0 & 0xFF);
        *h16 = fp16_of_int(q0);
      }
      return;
    }
    case 2:
      if (k == 2) {
        *a8 = s & 0xFF;
        *h16 = rot_exponent(pair_values[s & 15]) | (rot_exponent(pair_values[(s >> 4) & 15]) << 8);
      } else {
        *a8 = rot_exponent(s);
        *h16 = 0;
      }
      return;
    case 3:
      *a8 = s & 0xFF;
      *h16 = fp16_of_e4m3((uint8_t)s);
      return;
    default:
      *a8 = (uint32_t)((int32_t)s + value_offset) & 0xFF;
      *h16 = 0;
      return;
  }
}

}  // namespace ecw
