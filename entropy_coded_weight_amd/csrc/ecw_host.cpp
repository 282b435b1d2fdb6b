// Host side of the library: coding checks, histogram and frequency normalisation,
// the interleaved-tile rANS encoder, the blob writer and the blob validator.
//
// Method sources:
//  * frequencies minimise the cross-entropy size bound of the MINE page, Section
//    4.2 ("Compressed Size Prediction"): f_s >= 1 for every occurring symbol, sum M,
//    filled one unit at a time by largest marginal gain (exact for this separable
//    concave objective; ties to the smaller symbol);
//  * rANS with 32-bit states, 16-bit words, L = 2^16, at most one word per symbol,
//    independent tiles, per-tile start states and word offsets plus a final boundary
//    offset (EntroPack page, Sections 3.6 and C.3); encoding runs the decoder's
//    steps in reverse (MINE page, Section 3, "tANS");
//  * symbol maps: k integer codes per symbol (MINE page, Section 4.1), BF16 exponent
//    coded with the sign+mantissa byte raw (DFloat11 page, method section; MINE page
//    Section 4.1), FP8 bytes, E8 fields (EntroPack page, Sections 3.2, 3.3, A.3).
//  * validation before use, checked size arithmetic (quantized-artifact article,
//    loader validation section).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "ecw_internal.h"

namespace ecw {

static thread_local std::string g_last_error;

ecw_status fail(ecw_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}
void clear_error() { g_last_error.clear(); }

// ------------------------------------------------------------------ coding checks
ecw_status check_coding(const ecw_coding* c) {
  if (!c) return fail(ECW_E_INVALID_ARG, "coding is NULL");
  if (c->tile_rows != kLanes) return fail(ECW_E_UNSUPPORTED, "tile_rows must be 64");
  if (c->log2_m < kMinLog2M || c->log2_m > kMaxLog2M)
    return fail(ECW_E_UNSUPPORTED, "log2_m must be in [8, 13]");
  // E8 blocks are 8 columns wide and their tiles are not cut into 16-step groups:
  // any whole number of blocks per tile (so a tensor's tile count can be matched to
  // the device's wave slots); the other payloads stage 64 columns at a time
  const uint32_t tc_unit = c->payload == ECW_P_E8_LATTICE ? 8 : 64;
  if (c->tile_cols == 0 || c->tile_cols % tc_unit)
    return fail(ECW_E_INVALID_ARG, c->payload == ECW_P_E8_LATTICE ? "E8 tile_cols must be a positive multiple of 8"
                                                                   : "tile_cols must be a positive multiple of 64");
  if (c->rows > (1u << 30) || c->cols > (1u << 30))
    return fail(ECW_E_INVALID_ARG, "rows/cols too large");
  const bool quads = quad_coding(c->payload, c->code_bits, c->weights_per_symbol);
  if (!quads && c->stored_tuples != 0) return fail(ECW_E_INVALID_ARG, "stored_tuples is for INT quads of 4-bit codes");
  switch (c->payload) {
    case ECW_P_INT_CODES: {
      uint32_t b = c->code_bits, k = c->weights_per_symbol;
      if (b < 2 || b > 4) return fail(ECW_E_UNSUPPORTED, "code_bits must be 2, 3 or 4");
      if (quads) {
        // a table of stored 4-tuples; a record's column field has 11 bits
        if (c->stored_tuples < 1 || c->stored_tuples > std::min(kMaxTuples, 1u << c->log2_m))
          return fail(ECW_E_INVALID_ARG, "INT quads: stored_tuples must be in [1, min(M, 4096)]");
        if (c->tile_cols > 2048) return fail(ECW_E_UNSUPPORTED, "INT quads: tile_cols must be at most 2048");
      } else if (!(k == 1 || k == 2 || k == 4) || b * k > 8) {
        return fail(ECW_E_UNSUPPORTED, "weights_per_symbol must be 1, 2 or 4 with code_bits*k <= 8 "
                                       "(or 4 with 4-bit codes over stored tuples)");
      }
      if (!quads && (1u << (b * k)) > (1u << c->log2_m))
        return fail(ECW_E_UNSUPPORTED, "alphabet^k exceeds M (integer codes escape in quads of 4-bit codes only)");
      if (c->cols % (16 * k)) return fail(ECW_E_UNSUPPORTED, "cols must be a multiple of 16*k");
      if (c->recon_dtype != 0) return fail(ECW_E_INVALID_ARG, "recon_dtype is E8-only");
      break;
    }
    case ECW_P_BF16_EXP:
      if (c->weights_per_symbol == 2) {
        // exponent pairs with escapes; a record's column field has 11 bits
        if (c->cols % 32) return fail(ECW_E_UNSUPPORTED, "BF16 pairs: cols must be a multiple of 32");
        if (c->tile_cols > 2048) return fail(ECW_E_UNSUPPORTED, "BF16 pairs: tile_cols must be at most 2048");
      } else if (c->weights_per_symbol != 1) {
        return fail(ECW_E_UNSUPPORTED, "BF16 symbols carry one exponent or a pair");
      } else if (c->cols % 16) {
        return fail(ECW_E_UNSUPPORTED, "cols must be a multiple of 16");
      }
      if (c->recon_dtype != 0) return fail(ECW_E_INVALID_ARG, "recon_dtype is E8-only");
      break;
    case ECW_P_FP8_E4M3:
      if (c->weights_per_symbol != 1) return fail(ECW_E_UNSUPPORTED, "FP8 symbols carry one weight");
      if (c->cols % 16) return fail(ECW_E_UNSUPPORTED, "cols must be a multiple of 16");
      if (c->recon_dtype != 0) return fail(ECW_E_INVALID_ARG, "recon_dtype is E8-only");
      break;
    case ECW_P_E8_LATTICE:
      if (c->weights_per_symbol != 8) return fail(ECW_E_INVALID_ARG, "E8 blocks hold 8 weights");
      if (c->cols % 8) return fail(ECW_E_INVALID_ARG, "cols must be a multiple of 8");
      if (c->recon_dtype != ECW_DT_I8 && c->recon_dtype != ECW_DT_FP8_E4M3)
        return fail(ECW_E_INVALID_ARG, "E8 recon_dtype must be I8 or FP8_E4M3");
      break;
    default:
      return fail(ECW_E_INVALID_ARG, "unknown payload");
  }
  return ECW_OK;
}

Geometry geometry_of(const ecw_coding& c) {
  Geometry g{};
  g.n_tables = c.payload == ECW_P_E8_LATTICE ? 17 : 1;
  g.syms_per_row = symbols_per_row(c.payload, c.weights_per_symbol, c.cols);
  uint32_t sps = symbols_per_row_slice(c.payload, c.weights_per_symbol, c.tile_cols);
  g.n_rg = (c.rows + kLanes - 1) / kLanes;
  g.n_sl = g.syms_per_row ? (g.syms_per_row + sps - 1) / sps : 0;
  g.s_full = sps;
  g.s_last = g.n_sl ? g.syms_per_row - (g.n_sl - 1) * sps : 0;
  if (c.rows == 0) g.n_sl = 0, g.s_last = 0;
  g.n_tiles = g.n_rg * g.n_sl;
  return g;
}

// ------------------------------------------------------------------ symbol access
// Per row, the symbol stream in column order and (E8) its table index; BF16 also
// yields a raw byte per symbol.
struct Escape {
  uint32_t lane, col;     // col: column inside the tile's slice
  uint16_t bits;
};

// INT quads: how each of the 65536 tuples is coded.  A stored tuple is its own
// symbol; any other becomes the stored tuple reached by setting the fewest of its
// codes to 0 (position sets tried by count, then as a 4-bit mask ascending), and
// its nonzero codes so set are escaped.
struct QuadMap {
  std::vector<int32_t> id;     // symbol (index of the stored tuple), -1 = none
  std::vector<uint8_t> esc;    // bit i: code i is escaped

  void build(const uint16_t* stored, uint32_t n) {
    std::vector<int32_t> index(1u << 16, -1);
    for (uint32_t i = 0; i < n; ++i) index[stored[i]] = (int32_t)i;
    uint32_t order[15], no = 0;
    for (uint32_t pc = 1; pc <= 4; ++pc)
      for (uint32_t m = 1; m < 16; ++m)
        if ((uint32_t)__builtin_popcount(m) == pc) order[no++] = m;
    id.assign(1u << 16, -1);
    esc.assign(1u << 16, 0);
    for (uint32_t v = 0; v < (1u << 16); ++v) {
      if (index[v] >= 0) {
        id[v] = index[v];
        continue;
      }
      for (uint32_t oi = 0; oi < 15; ++oi) {
        const uint32_t m = order[oi];
        uint32_t z = v, e = 0;
        for (uint32_t p = 0; p < 4; ++p)
          if ((m >> p) & 1) {
            if (((v >> (4 * p)) & 15) != 8) e |= 1u << p;
            z = (z & ~(15u << (4 * p))) | (8u << (4 * p));
          }
        if (index[z] >= 0) {
          id[v] = index[z];
          esc[v] = (uint8_t)e;
          break;
        }
      }
    }
  }
};

// bf16 bits of a small integer (exact)
static uint16_t bf16_of_int(int q) {
  const float f = (float)q;
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

struct SymbolSource {
  const ecw_coding& c;
  const void* w;
  const ecw_tables* t;   // value offsets (E8); may be null while building tables
  int8_t digit[256];     // BF16 pairs: digit of each exponent, -1 = escaped
  const QuadMap* qm = nullptr;   // INT quads

  // BF16 pairs: exponent 0 has digit 0; e != 0 the first d >= 1 with pv[d] == e.
  void set_digits(const uint8_t* pv) {
    for (int e = 0; e < 256; ++e) digit[e] = -1;
    for (int d = (int)kPairDigits - 1; d >= 1; --d)
      if (pv[d]) digit[pv[d]] = (int8_t)d;
    digit[0] = 0;
  }

  // Writes n symbols of row r starting at symbol index s0.  Returns false on an
  // invalid logical value.  tbl/raw may be null; raw gets one byte per weight.
  // BF16 pairs: escaped weights get raw byte 0 and, if esc is given, an Escape
  // (lane `lane`, column relative to symbol s0's first column); INT quads likewise
  // (the escaped code reads as 0).
  bool row(uint32_t r, uint32_t s0, uint32_t n, int32_t* val, uint8_t* tbl, uint8_t* raw,
           std::vector<Escape>* esc = nullptr, uint32_t lane = 0) const {
    const uint64_t K = c.cols;
    switch (c.payload) {
      case ECW_P_INT_CODES: {
        const int8_t* q = static_cast<const int8_t*>(w) + r * K;
        const uint32_t b = c.code_bits, k = c.weights_per_symbol;
        const int half = 1 << (b - 1);
        for (uint32_t i = 0; i < n; ++i) {
          uint32_t s = 0;
          for (uint32_t u = 0; u < k; ++u) {
            int v = q[(uint64_t)(s0 + i) * k + u];
            if (v < -half || v >= half) return false;
            s |= (uint32_t)(v + half) << (b * u);
          }
          if (qm) {
            const int32_t id = qm->id[s];
            if (id < 0) return false;
            if (esc && qm->esc[s])
              for (uint32_t u = 0; u < 4; ++u)
                if ((qm->esc[s] >> u) & 1)
                  esc->push_back({lane, 4 * i + u, bf16_of_int(q[(uint64_t)(s0 + i) * 4 + u])});
            s = (uint32_t)id;
          }
          val[i] = (int32_t)s;
          if (tbl) tbl[i] = 0;
        }
        return true;
      }
      case ECW_P_BF16_EXP: {
        const uint16_t* p = static_cast<const uint16_t*>(w) + r * K;
        if (c.weights_per_symbol == 2) {
          for (uint32_t i = 0; i < n; ++i) {
            uint32_t s = 0;
            for (uint32_t u = 0; u < 2; ++u) {
              const uint32_t col = 2 * (s0 + i) + u;
              const uint16_t bits = p[col];
              int d = digit[(bits >> 7) & 0xFF];
              uint8_t rb = (uint8_t)(((bits >> 8) & 0x80) | (bits & 0x7F));
              if (d < 0) {
                d = 0;
                rb = 0;
                if (esc) esc->push_back({lane, 2 * i + u, bits});
              }
              s |= (uint32_t)d << (4 * u);
              if (raw) raw[2 * i + u] = rb;
            }
            val[i] = (int32_t)s;
            if (tbl) tbl[i] = 0;
          }
          return true;
        }
        for (uint32_t i = 0; i < n; ++i) {
          uint32_t bits = p[s0 + i];
          val[i] = (int32_t)((bits >> 7) & 0xFF);
          if (tbl) tbl[i] = 0;
          if (raw) raw[i] = (uint8_t)(((bits >> 8) & 0x80) | (bits & 0x7F));
        }
        return true;
      }
      case ECW_P_FP8_E4M3: {
        const uint8_t* p = static_cast<const uint8_t*>(w) + r * K;
        for (uint32_t i = 0; i < n; ++i) {
          val[i] = p[s0 + i];
          if (tbl) tbl[i] = 0;
        }
        return true;
      }
      case ECW_P_E8_LATTICE: {
        // s0 and n are multiples of 9 (slices hold whole blocks)
        const int8_t* v2 = static_cast<const int8_t*>(w) + r * K;
        for (uint32_t blk = 0; blk < n / 9; ++blk) {
          const int8_t* p = v2 + (uint64_t)(s0 / 9 + blk) * 8;
          int c0 = p[0] & 1;
          int z[8];
          int zsum = 0;
          for (int i = 0; i < 8; ++i) {
            if ((p[i] & 1) != c0) return false;
            z[i] = (p[i] - c0) / 2;
            zsum += z[i];
          }
          if (zsum & 1) return false;
          int32_t* o = val + blk * 9;
          o[0] = c0;
          for (int i = 0; i < 7; ++i) o[1 + i] = z[i];
          o[8] = (z[7] >= 0) ? z[7] / 2 : -((-z[7] + 1) / 2);   // floor(z8 / 2)
          if (tbl) {
            uint8_t* tt = tbl + blk * 9;
            tt[0] = 0;
            for (int j = 1; j < 9; ++j) tt[j] = (uint8_t)(1 + 8 * c0 + (j - 1));
          }
        }
        return true;
      }
    }
    return false;
  }
};

static unsigned n_threads() {
  unsigned h = std::thread::hardware_concurrency();
  return std::max(1u, std::min(h ? h : 1u, 64u));
}

template <class F>
static void parallel_for(uint64_t n, F&& f) {
  unsigned nt = (unsigned)std::min<uint64_t>(n_threads(), std::max<uint64_t>(n, 1));
  if (nt <= 1) {
    for (uint64_t i = 0; i < n; ++i) f(i, 0u);
    return;
  }
  std::atomic<uint64_t> next{0};
  std::vector<std::thread> th;
  for (unsigned t = 0; t < nt; ++t)
    th.emplace_back([&, t] {
      for (;;) {
        uint64_t i = next.fetch_add(1);
        if (i >= n) break;
        f(i, t);
      }
    });
  for (auto& x : th) x.join();
}

// ------------------------------------------------------------------ normaliser
// A symbols (256, or the stored tuples of INT quads); at most M of them occur.
static void normalise(const uint64_t* count, uint32_t A, uint32_t log2_m, uint16_t* freq) {
  const uint32_t M = 1u << log2_m;
  uint32_t present = 0;
  for (uint32_t s = 0; s < A; ++s) present += count[s] > 0;
  for (uint32_t s = 0; s < A; ++s) freq[s] = 0;
  if (present == 0) return;
  if (present == 1) {
    for (uint32_t s = 0; s < A; ++s)
      if (count[s]) freq[s] = (uint16_t)M;
    return;
  }
  std::vector<double> d(M + 1, 0.0);
  for (uint32_t f = 1; f <= M; ++f) d[f] = std::log2((double)f + 1.0) - std::log2((double)f);
  std::vector<uint32_t> f(A);
  std::vector<double> gain(A);
  for (uint32_t s = 0; s < A; ++s) {
    f[s] = count[s] ? 1 : 0;
    gain[s] = count[s] ? (double)count[s] * d[1] : -INFINITY;
  }
  for (uint32_t it = 0; it < M - present; ++it) {
    uint32_t best = 0;
    for (uint32_t s = 1; s < A; ++s)
      if (gain[s] > gain[best]) best = s;        // strict: first maximum wins
    f[best] += 1;
    gain[best] = (double)count[best] * d[f[best]];
  }
  for (uint32_t s = 0; s < A; ++s) freq[s] = (uint16_t)f[s];
}

}  // namespace ecw

using namespace ecw;

extern "C" uint32_t ecw_abi_version(void) { return ECW_ABI_VERSION; }
extern "C" const char* ecw_last_error(void) { return g_last_error.c_str(); }

// ------------------------------------------------------------------ enc_e8_nearest
namespace ecw {

// Nearest point of D8 (integer vectors with an even sum) to y: round each
// coordinate half to even; if the sum is odd, round the coordinate with the largest
// rounding error (lowest index on ties) the other way.
static void nearest_d8(const double* y, double* z) {
  double sum = 0.0;
  int worst = 0;
  double worst_err = -1.0;
  for (int i = 0; i < 8; ++i) {
    z[i] = std::nearbyint(y[i]);
    sum += z[i];
    const double e = std::fabs(y[i] - z[i]);
    if (e > worst_err) {
      worst_err = e;
      worst = i;
    }
  }
  if (std::fmod(sum, 2.0) != 0.0) z[worst] += (y[worst] - z[worst] >= 0.0) ? 1.0 : -1.0;
}

// Squared distance, summed as pairs of pairs (((d0+d1)+(d2+d3))+((d4+d5)+(d6+d7))).
static double dist2(const double* y, const double* p, double shift) {
  double d[8];
  for (int i = 0; i < 8; ++i) {
    const double t = y[i] - (p[i] + shift);
    d[i] = t * t;
  }
  return ((d[0] + d[1]) + (d[2] + d[3])) + ((d[4] + d[5]) + (d[6] + d[7]));
}

}  // namespace ecw

extern "C" ecw_status enc_e8_nearest(const double* u, size_t n_blocks, int8_t* v2) {
  clear_error();
  if (n_blocks && (!u || !v2)) return fail(ECW_E_INVALID_ARG, "NULL input or output");
  std::vector<int8_t> out(n_blocks * 8);
  for (size_t b = 0; b < n_blocks; ++b) {
    const double* y = u + b * 8;
    double z0[8], z1[8], ym[8];
    for (int i = 0; i < 8; ++i) {
      if (!std::isfinite(y[i])) return fail(ECW_E_INVALID_ARG, "non-finite input");
      ym[i] = y[i] - 0.5;
    }
    nearest_d8(y, z0);
    nearest_d8(ym, z1);
    const bool half = dist2(y, z1, 0.5) < dist2(y, z0, 0.0);
    for (int i = 0; i < 8; ++i) {
      const double d = half ? 2.0 * z1[i] + 1.0 : 2.0 * z0[i];
      if (d < -127.0 || d > 127.0) return fail(ECW_E_UNSUPPORTED, "doubled coordinate outside int8");
      out[b * 8 + i] = (int8_t)d;
    }
  }
  if (n_blocks) std::memcpy(v2, out.data(), out.size());
  return ECW_OK;
}

// ------------------------------------------------------------------ enc_build_tables
extern "C" ecw_status enc_build_tables(const ecw_coding* c, const void* w, ecw_tables* out) {
  clear_error();
  ecw_status st = check_coding(c);
  if (st != ECW_OK) return st;
  if (!out) return fail(ECW_E_INVALID_ARG, "tables output is NULL");
  if (!w && c->rows && c->cols) return fail(ECW_E_INVALID_ARG, "weights are NULL");
  Geometry g = geometry_of(*c);
  std::memset(out, 0, sizeof(*out));
  out->n_tables = g.n_tables;
  const uint32_t nth = n_threads();
  std::vector<std::vector<uint64_t>> hist(nth, std::vector<uint64_t>(17 * 512, 0));
  std::vector<int32_t> vmin(nth * 17, INT32_MAX), vmax(nth * 17, INT32_MIN);
  std::atomic<bool> bad{false};
  SymbolSource src{*c, w, nullptr, {}};
  if (quad_coding(c->payload, c->code_bits, c->weights_per_symbol)) {
    // INT quads: the stored_tuples most frequent 4-tuples (ties to the smaller
    // tuple, the zero tuple always kept in place of the last), ascending (MINE page,
    // Section 4.1 "Escapes", Section 4.2 "Tuning t")
    std::vector<std::vector<uint64_t>> th(nth);
    parallel_for(c->rows, [&](uint64_t r, unsigned tid) {
      if (th[tid].empty()) th[tid].assign(1u << 16, 0);
      const int8_t* q = static_cast<const int8_t*>(w) + r * (uint64_t)c->cols;
      uint64_t* h = th[tid].data();
      for (uint32_t j = 0; j < c->cols / 4; ++j) {
        uint32_t v = 0;
        for (uint32_t u = 0; u < 4; ++u) {
          const int x = q[4 * j + u];
          if (x < -8 || x > 7) {
            bad = true;
            return;
          }
          v |= (uint32_t)(x + 8) << (4 * u);
        }
        h[v] += 1;
      }
    });
    if (bad) return fail(ECW_E_INVALID_ARG, "logical tensor holds a value outside the payload's range");
    std::vector<uint64_t> cnt(1u << 16, 0);
    for (auto& h : th)
      if (!h.empty())
        for (uint32_t v = 0; v < (1u << 16); ++v) cnt[v] += h[v];
    std::vector<uint32_t> order;
    for (uint32_t v = 0; v < (1u << 16); ++v)
      if (cnt[v]) order.push_back(v);
    std::sort(order.begin(), order.end(), [&](uint32_t a, uint32_t b) { return cnt[a] != cnt[b] ? cnt[a] > cnt[b] : a < b; });
    order.resize(std::min<size_t>(order.size(), c->stored_tuples));
    if (std::find(order.begin(), order.end(), kQuadZero) == order.end()) {
      if (order.size() == c->stored_tuples) order.pop_back();
      order.push_back(kQuadZero);
    }
    std::sort(order.begin(), order.end());
    out->n_tuples = (uint32_t)order.size();
    for (size_t i = 0; i < order.size(); ++i) out->tuples[i] = (uint16_t)order[i];
    QuadMap qm;
    qm.build(out->tuples, out->n_tuples);
    for (uint32_t v = 0; v < (1u << 16); ++v) {
      if (!cnt[v]) continue;
      out->tuple_count[qm.id[v]] += cnt[v];
      out->escapes += cnt[v] * (uint64_t)__builtin_popcount(qm.esc[v]);
    }
    out->alphabet[0] = out->n_tuples;
    normalise(out->tuple_count, out->n_tuples, c->log2_m, out->tuple_freq);
    return ECW_OK;
  }
  if (c->payload == ECW_P_BF16_EXP && c->weights_per_symbol == 2) {
    // BF16 pairs: the stored exponents are 0 and the 15 most frequent others, the
    // smaller exponent first on ties, ascending (MINE page, Section 4.2 "Tuning t")
    std::vector<std::vector<uint64_t>> eh(nth, std::vector<uint64_t>(256, 0));
    parallel_for(c->rows, [&](uint64_t r, unsigned tid) {
      const uint16_t* p = static_cast<const uint16_t*>(w) + r * (uint64_t)c->cols;
      uint64_t* h = eh[tid].data();
      for (uint32_t i = 0; i < c->cols; ++i) h[(p[i] >> 7) & 0xFF] += 1;
    });
    uint64_t ec[256] = {0};
    for (uint32_t k = 0; k < nth; ++k)
      for (int e = 0; e < 256; ++e) ec[e] += eh[k][e];
    std::vector<uint32_t> order;
    for (uint32_t e = 1; e < 256; ++e)
      if (ec[e]) order.push_back(e);
    std::sort(order.begin(), order.end(), [&](uint32_t a, uint32_t b) { return ec[a] != ec[b] ? ec[a] > ec[b] : a < b; });
    order.resize(std::min<size_t>(order.size(), kPairDigits - 1));
    std::sort(order.begin(), order.end());
    for (size_t i = 0; i < order.size(); ++i) out->pair_values[1 + i] = (uint8_t)order[i];
    src.set_digits(out->pair_values);
    for (int e = 0; e < 256; ++e)
      if (src.digit[e] < 0) out->escapes += ec[e];
  }
  // E8 values are offset by 256 inside the scratch histogram so negatives index it
  parallel_for(c->rows, [&](uint64_t r, unsigned tid) {
    std::vector<int32_t> val(g.syms_per_row);
    std::vector<uint8_t> tbl(g.syms_per_row);
    if (!src.row((uint32_t)r, 0, g.syms_per_row, val.data(), tbl.data(), nullptr)) {
      bad = true;
      return;
    }
    uint64_t* h = hist[tid].data();
    for (uint32_t i = 0; i < g.syms_per_row; ++i) {
      int32_t v = val[i];
      uint32_t t = tbl[i];
      if (v < -256 || v > 255) {
        bad = true;
        return;
      }
      h[t * 512 + (uint32_t)(v + 256)] += 1;
      vmin[tid * 17 + t] = std::min(vmin[tid * 17 + t], v);
      vmax[tid * 17 + t] = std::max(vmax[tid * 17 + t], v);
    }
  });
  if (bad) return fail(ECW_E_INVALID_ARG, "logical tensor holds a value outside the payload's range");
  for (uint32_t t = 0; t < g.n_tables; ++t) {
    int32_t lo = INT32_MAX, hi = INT32_MIN;
    for (uint32_t k = 0; k < nth; ++k) {
      lo = std::min(lo, vmin[k * 17 + t]);
      hi = std::max(hi, vmax[k * 17 + t]);
    }
    int32_t off = 0;
    uint32_t alpha = 0;
    if (c->payload == ECW_P_E8_LATTICE) {
      if (lo <= hi) {
        off = lo;
        alpha = (uint32_t)(hi - lo + 1);
      }
      if (alpha > 256) return fail(ECW_E_UNSUPPORTED, "E8 field alphabet larger than 256");
    } else if (c->payload == ECW_P_INT_CODES) {
      alpha = 1u << (c->code_bits * c->weights_per_symbol);
    } else {
      alpha = 256;
    }
    out->alphabet[t] = alpha;
    out->value_offset[t] = off;
    uint64_t present = 0;
    for (uint32_t s = 0; s < 256; ++s) {
      int32_t v = (int32_t)s + off;
      uint64_t n = 0;
      if (v >= -256 && v <= 255)
        for (uint32_t k = 0; k < nth; ++k) n += hist[k][t * 512 + (uint32_t)(v + 256)];
      out->count[t][s] = s < alpha ? n : 0;
      present += out->count[t][s] > 0;
    }
    if (present > (1u << c->log2_m))
      return fail(ECW_E_UNSUPPORTED, "more distinct symbols than table slots (only BF16 exponent pairs escape)");
    normalise(out->count[t], 256, c->log2_m, out->freq[t]);
  }
  return ECW_OK;
}

// ------------------------------------------------------------------ enc_encode
namespace {

struct TileOut {
  std::vector<uint16_t> words;   // decoder order
  uint32_t states[64];
};

struct Lut {
  std::vector<uint32_t> cum;     // [n_tables][256]
};

}  // namespace

static uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

static ecw_status check_tables_for(const ecw_coding* c, const ecw_tables* t, const Geometry& g) {
  if (!t) return fail(ECW_E_INVALID_ARG, "tables are NULL");
  if (t->n_tables != g.n_tables) return fail(ECW_E_INVALID_ARG, "table count does not match payload");
  const uint32_t M = 1u << c->log2_m;
  const bool quads = quad_coding(c->payload, c->code_bits, c->weights_per_symbol);
  for (uint32_t k = 0; k < g.n_tables && !quads; ++k) {
    if (t->alphabet[k] > 256) return fail(ECW_E_INVALID_ARG, "alphabet > 256");
    uint64_t sum = 0;
    for (uint32_t s = 0; s < 256; ++s) {
      if (s >= t->alphabet[k] && t->freq[k][s]) return fail(ECW_E_INVALID_ARG, "freq beyond alphabet");
      sum += t->freq[k][s];
    }
    if (sum != M && !(sum == 0 && g.n_tiles == 0) && !(sum == 0 && c->payload == ECW_P_E8_LATTICE))
      return fail(ECW_E_INVALID_ARG, "table frequencies do not sum to M");
  }
  if (c->payload == ECW_P_BF16_EXP && c->weights_per_symbol == 2 && t->pair_values[0] != 0)
    return fail(ECW_E_INVALID_ARG, "BF16 pairs: digit 0 must be exponent 0 (escaped weights are coded as 0)");
  if (quads) {
    const uint32_t n = t->n_tuples;
    if (n < 1 || n > c->stored_tuples) return fail(ECW_E_INVALID_ARG, "INT quads: n_tuples must be in [1, stored_tuples]");
    bool zero = false;
    uint64_t sum = 0;
    for (uint32_t i = 0; i < n; ++i) {
      if (i && t->tuples[i] <= t->tuples[i - 1]) return fail(ECW_E_INVALID_ARG, "INT quads: tuples not ascending");
      zero |= t->tuples[i] == kQuadZero;
      sum += t->tuple_freq[i];
    }
    if (!zero) return fail(ECW_E_INVALID_ARG, "INT quads: the zero tuple must be stored (escapes are coded as 0)");
    if (sum != M && !(sum == 0 && g.n_tiles == 0)) return fail(ECW_E_INVALID_ARG, "tuple frequencies do not sum to M");
  }
  return ECW_OK;
}

extern "C" ecw_status enc_encode(const ecw_coding* c, const ecw_tables* t, const void* w,
                                 const uint16_t* row_scales, void* blob, size_t* blob_bytes) {
  clear_error();
  ecw_status st = check_coding(c);
  if (st != ECW_OK) return st;
  if (!blob_bytes) return fail(ECW_E_INVALID_ARG, "blob_bytes is NULL");
  Geometry g = geometry_of(*c);
  st = check_tables_for(c, t, g);
  if (st != ECW_OK) return st;
  const bool has_scales = c->payload != ECW_P_BF16_EXP;
  if (has_scales && !row_scales && c->rows) return fail(ECW_E_INVALID_ARG, "row scales are NULL");
  if (!w && c->rows && c->cols) return fail(ECW_E_INVALID_ARG, "weights are NULL");
  const uint32_t M = 1u << c->log2_m;
  const uint32_t m = c->log2_m;
  const bool bf16 = c->payload == ECW_P_BF16_EXP;
  const bool pairs = bf16 && c->weights_per_symbol == 2;
  const bool quads = quad_coding(c->payload, c->code_bits, c->weights_per_symbol);
  const bool escapes = pairs || quads;
  const uint32_t kw = bf16 ? c->weights_per_symbol : 1;     // raw bytes per symbol
  SymbolSource src0{*c, w, t, {}};
  if (pairs) src0.set_digits(t->pair_values);
  QuadMap qm;
  if (quads) {
    qm.build(t->tuples, t->n_tuples);
    src0.qm = &qm;
  }
  // symbols per table: 256, or the stored tuples
  const uint32_t A = quads ? t->n_tuples : 256;

  // Section sizes that do not depend on the coded words
  const uint64_t tables_b = (uint64_t)g.n_tables * sizeof(TableRecord) + (pairs ? kPairDigits : 0) +
                            (quads ? 4ull * c->stored_tuples : 0);
  const uint64_t lut_b = (uint64_t)g.n_tables * M * 8;
  const uint64_t states_b = (uint64_t)g.n_tiles * 64 * 4;
  const uint64_t offsets_b = ((uint64_t)g.n_tiles + 1) * 4;
  uint64_t raw_b = 0;
  if (bf16) {
    for (uint32_t sl = 0; sl < g.n_sl; ++sl) {
      uint32_t S = (sl + 1 == g.n_sl) ? g.s_last : g.s_full;
      raw_b += raw_group_count(S * kw) * 1024ull * g.n_rg;
    }
  }
  const uint64_t scales_b = has_scales ? (uint64_t)c->rows * 2 : 0;
  uint64_t max_words = (uint64_t)g.n_rg * 64 * g.syms_per_row;   // <= 1 word per symbol
  if (pairs) {
    // correction streams: a 4-word mask per tile and 2 words per escaped weight
    std::atomic<uint64_t> n_esc{0};
    if (w)
      parallel_for(c->rows, [&](uint64_t r, unsigned) {
        const uint16_t* p = static_cast<const uint16_t*>(w) + r * (uint64_t)c->cols;
        uint64_t n = 0;
        for (uint32_t i = 0; i < c->cols; ++i) n += src0.digit[(p[i] >> 7) & 0xFF] < 0;
        n_esc += n;
      });
    max_words += (uint64_t)g.n_tiles * kEscMaskWords + 2 * n_esc.load();
  }
  if (quads) {
    std::atomic<uint64_t> n_esc{0};
    if (w)
      parallel_for(c->rows, [&](uint64_t r, unsigned) {
        const int8_t* q = static_cast<const int8_t*>(w) + r * (uint64_t)c->cols;
        uint64_t n = 0;
        for (uint32_t j = 0; j < c->cols / 4; ++j) {
          uint32_t v = 0;
          for (uint32_t u = 0; u < 4; ++u) v |= (uint32_t)((q[4 * j + u] + 8) & 15) << (4 * u);
          n += (uint64_t)__builtin_popcount(qm.esc[v]);
        }
        n_esc += n;
      });
    max_words += (uint64_t)g.n_tiles * kEscMaskWords + 2 * n_esc.load();
  }
  auto layout = [&](uint64_t n_words, SectionRef* sec) {
    uint64_t pos = kHeaderBytes;
    const uint64_t sizes[kNumSections] = {tables_b, lut_b, states_b, offsets_b,
                                          n_words * 2 + kWordPad, raw_b, scales_b};
    for (int s = 0; s < (int)kNumSections; ++s) {
      pos = align_up(pos, kSectionAlign);
      sec[s].offset = pos;
      sec[s].bytes = sizes[s];
      pos += sizes[s];
    }
    return align_up(pos, kSectionAlign);
  };
  SectionRef tmp[kNumSections];
  const uint64_t bound = layout(max_words, tmp);
  if (!blob) {
    *blob_bytes = (size_t)bound;   // upper bound; the filling call reports the exact size
    return ECW_OK;
  }

  // frequencies and cumulative frequencies, A per table
  std::vector<uint32_t> fr((size_t)g.n_tables * A, 0), cum((size_t)g.n_tables * A, 0);
  for (uint32_t k = 0; k < g.n_tables; ++k) {
    uint32_t a = 0;
    for (uint32_t s = 0; s < A; ++s) {
      fr[k * A + s] = quads ? t->tuple_freq[s] : t->freq[k][s];
      cum[k * A + s] = a;
      a += fr[k * A + s];
    }
  }

  // Encode every tile (independent) on all host threads.
  std::vector<TileOut> tiles(g.n_tiles);
  std::atomic<bool> bad_value{false}, bad_freq{false};
  std::vector<uint8_t> raw_plane(raw_b, 0);
  parallel_for(g.n_tiles, [&](uint64_t ti, unsigned) {
    const uint32_t rg = (uint32_t)(ti / g.n_sl), sl = (uint32_t)(ti % g.n_sl);
    const uint32_t S = (sl + 1 == g.n_sl) ? g.s_last : g.s_full;
    const uint32_t s0 = sl * g.s_full;
    std::vector<int32_t> val((size_t)64 * S);
    std::vector<uint8_t> tbl((size_t)64 * S);
    std::vector<Escape> esc;   // BF16 pairs, lanes ascending, columns ascending
    bool active[64];
    const SymbolSource& src = src0;
    for (uint32_t l = 0; l < 64; ++l) {
      uint32_t r = rg * 64 + l;
      active[l] = r < c->rows;
      if (!active[l]) continue;
      if (!src.row(r, s0, S, &val[(size_t)l * S], &tbl[(size_t)l * S], nullptr, escapes ? &esc : nullptr, l)) {
        bad_value = true;
        return;
      }
    }
    // symbols relative to the table's value offset
    for (uint32_t l = 0; l < 64; ++l) {
      if (!active[l]) continue;
      for (uint32_t j = 0; j < S; ++j) {
        int32_t s = val[(size_t)l * S + j] - t->value_offset[tbl[(size_t)l * S + j]];
        if (s < 0 || (uint32_t)s >= A) {
          bad_value = true;
          return;
        }
        val[(size_t)l * S + j] = s;
      }
    }
    TileOut& o = tiles[ti];
    uint64_t x[64];
    for (int l = 0; l < 64; ++l) x[l] = kStateL;
    std::vector<uint16_t> pushed;
    pushed.reserve((size_t)64 * S / 2 + 64);
    for (int64_t j = (int64_t)S - 1; j >= 0; --j) {
      for (int l = 63; l >= 0; --l) {
        if (!active[l]) continue;
        const uint32_t tb = tbl[(size_t)l * S + j];
        const uint32_t s = (uint32_t)val[(size_t)l * S + j];
        const uint64_t f = fr[tb * A + s];
        if (f == 0) {
          bad_freq = true;
          return;
        }
        const uint64_t x_max = f << (32 - m);   // ((L >> m) << 16) * f
        if (x[l] >= x_max) {
          pushed.push_back((uint16_t)(x[l] & 0xFFFF));
          x[l] >>= 16;
        }
        x[l] = (x[l] / f) * M + (x[l] % f) + cum[tb * A + s];
      }
    }
    o.words.assign(pushed.rbegin(), pushed.rend());
    for (int l = 0; l < 64; ++l) o.states[l] = (uint32_t)x[l];
    if (escapes) {
      // correction stream after the ANS words: lane mask, then rounds of records
      uint32_t cnt[64] = {0}, first[64] = {0}, rounds = 0;
      uint64_t mask = 0;
      for (const Escape& e : esc) ++cnt[e.lane];
      for (uint32_t l = 0, a = 0; l < 64; ++l) {
        first[l] = a;
        a += cnt[l];
        if (cnt[l]) mask |= 1ull << l;
        rounds = std::max(rounds, cnt[l]);
      }
      for (uint32_t i = 0; i < kEscMaskWords; ++i) o.words.push_back((uint16_t)(mask >> (16 * i)));
      for (uint32_t rd = 0; rd < rounds; ++rd)
        for (uint32_t l = 0; l < 64; ++l) {
          if (cnt[l] <= rd) continue;
          const Escape& e = esc[first[l] + rd];
          const uint32_t rec = e.bits | (e.col << 16) | (rd + 1 == cnt[l] ? kEscLast : 0u);
          o.words.push_back((uint16_t)rec);
          o.words.push_back((uint16_t)(rec >> 16));
        }
    }
  });
  if (bad_value) return fail(ECW_E_INVALID_ARG, "logical tensor holds a value outside the tables");
  if (bad_freq) return fail(ECW_E_INVALID_ARG, "a symbol of the tensor has zero frequency");

  // BF16 raw plane (row-group-major tile order), written serially per tile
  if (bf16) {
    uint64_t pos = 0;
    const SymbolSource& src = src0;
    std::vector<int32_t> val;
    std::vector<uint8_t> raw;
    for (uint32_t ti = 0; ti < g.n_tiles; ++ti) {
      const uint32_t rg = ti / g.n_sl, sl = ti % g.n_sl;
      const uint32_t S = (sl + 1 == g.n_sl) ? g.s_last : g.s_full;
      const uint32_t nw = S * kw;             // weights per lane
      const uint64_t G = raw_group_count(nw);
      val.resize(S);
      raw.resize(nw);
      for (uint32_t l = 0; l < 64; ++l) {
        uint32_t r = rg * 64 + l;
        if (r >= c->rows) continue;
        src.row(r, sl * g.s_full, S, val.data(), nullptr, raw.data());
        for (uint32_t j = 0; j < nw; ++j) raw_plane[pos + (j / 16) * 1024 + l * 16 + (j % 16)] = raw[j];
      }
      pos += G * 1024;
    }
  }

  uint64_t n_words = 0;
  for (auto& o : tiles) n_words += o.words.size();
  if (n_words > 0xFFFFFFFFull) return fail(ECW_E_UNSUPPORTED, "tensor needs more than 2^32 words");
  SectionRef sec[kNumSections];
  const uint64_t total = layout(n_words, sec);
  if (*blob_bytes < total) {
    *blob_bytes = (size_t)total;
    return fail(ECW_E_BUFFER_TOO_SMALL, "blob buffer too small");
  }
  uint8_t* out = static_cast<uint8_t*>(blob);
  std::memset(out, 0, total);
  BlobHeader h{};
  h.magic = kMagic;
  h.version = kVersion;
  h.header_bytes = kHeaderBytes;
  h.n_sections = kNumSections;
  h.payload = c->payload;
  h.rows = c->rows;
  h.cols = c->cols;
  h.weights_per_symbol = c->weights_per_symbol;
  h.code_bits = c->code_bits;
  h.log2_m = c->log2_m;
  h.tile_rows = c->tile_rows;
  h.tile_cols = c->tile_cols;
  h.recon_dtype = c->recon_dtype;
  h.stored_tuples = c->stored_tuples;
  h.n_tables = g.n_tables;
  h.n_row_groups = g.n_rg;
  h.n_slices = g.n_sl;
  h.n_tiles = g.n_tiles;
  h.steps_full = g.s_full;
  h.steps_last = g.s_last;
  h.lut_entry_bytes = 8;
  h.total_bytes = total;
  for (int s = 0; s < (int)kNumSections; ++s) h.sec[s] = sec[s];
  std::memcpy(out, &h, sizeof(h));

  // TABLES and LUT
  for (uint32_t k = 0; k < g.n_tables; ++k) {
    TableRecord rec{};
    rec.alphabet = quads ? t->n_tuples : t->alphabet[k];
    rec.value_offset = t->value_offset[k];
    if (!quads) std::memcpy(rec.freq, t->freq[k], sizeof(rec.freq));
    std::memcpy(out + sec[kSecTables].offset + k * sizeof(TableRecord), &rec, sizeof(rec));
    uint32_t* lut = reinterpret_cast<uint32_t*>(out + sec[kSecLut].offset) + (size_t)k * M * 2;
    uint32_t slot = 0;
    for (uint32_t s = 0; s < A; ++s) {
      const uint32_t f = fr[k * A + s];
      if (quads) {
        for (uint32_t i = 0; i < f; ++i, ++slot) quad_entry(f, i, t->tuples[s], &lut[2 * slot], &lut[2 * slot + 1]);
        continue;
      }
      uint32_t a8 = 0, h16 = 0;
      entry_payload(c->payload, c->code_bits, c->weights_per_symbol, t->value_offset[k], t->pair_values, s, &a8,
                    &h16);
      for (uint32_t i = 0; i < f; ++i, ++slot) {
        lut[2 * slot] = f | (a8 << 24);
        lut[2 * slot + 1] = i | (h16 << 16);   // bias = slot - cum[s]
      }
    }
  }
  if (pairs) std::memcpy(out + sec[kSecTables].offset + g.n_tables * sizeof(TableRecord), t->pair_values, kPairDigits);
  if (quads) {
    uint8_t* q = out + sec[kSecTables].offset + sizeof(TableRecord);
    std::memcpy(q, t->tuples, 2ull * t->n_tuples);
    std::memcpy(q + 2ull * c->stored_tuples, t->tuple_freq, 2ull * t->n_tuples);
  }
  // STATES, OFFSETS, WORDS
  uint32_t* states = reinterpret_cast<uint32_t*>(out + sec[kSecStates].offset);
  uint32_t* offs = reinterpret_cast<uint32_t*>(out + sec[kSecOffsets].offset);
  uint16_t* words = reinterpret_cast<uint16_t*>(out + sec[kSecWords].offset);
  uint64_t wpos = 0;
  for (uint32_t ti = 0; ti < g.n_tiles; ++ti) {
    std::memcpy(states + (size_t)ti * 64, tiles[ti].states, 256);
    offs[ti] = (uint32_t)wpos;
    if (!tiles[ti].words.empty())
      std::memcpy(words + wpos, tiles[ti].words.data(), tiles[ti].words.size() * 2);
    wpos += tiles[ti].words.size();
  }
  offs[g.n_tiles] = (uint32_t)wpos;
  if (raw_b) std::memcpy(out + sec[kSecRaw].offset, raw_plane.data(), raw_b);
  if (scales_b) std::memcpy(out + sec[kSecScales].offset, row_scales, scales_b);
  *blob_bytes = (size_t)total;
  return ECW_OK;
}

// ------------------------------------------------------------------ dec_prepare
namespace ecw {

// Default launch shape: one tile per wave, up to 16 waves (consecutive slices of
// one row group) per block, halved until the block's LDS (decode tables, staged
// activations at batch capacity 4, word rings) fits the CU's 160 KiB.  Per-tensor
// tuning may change it.
void default_launch(ecw_tensor* t) {
  const uint32_t n_sl = t->n_slices;
  t->tiles_per_wave = 1;
  t->streams_per_wave = 1;
  t->row_groups_per_block = 1;
  uint32_t W = std::max(1u, std::min(16u, n_sl));
  while (W > 1 && launch_lds_bytes(t, W, 1, 4, false, true) > 160u * 1024u) W /= 2;
  t->waves_per_block = W;
}

uint32_t slice_groups(const ecw_tensor* t) {
  const uint32_t per = t->waves_per_block * t->tiles_per_wave;
  return per ? (t->n_slices + per - 1) / per : 0;
}

uint64_t partial_bytes(const ecw_tensor* t, int batch) {
  const uint32_t nsg = slice_groups(t);
  if (nsg <= 1) return 0;
  const uint64_t B = batch > 1 ? 4 : 1;   // kernels are built for batch capacity 1 or 4
  return align_up((uint64_t)t->n_row_groups * nsg * B * 64 * 4, 256);
}

uint64_t ticket_bytes(const ecw_tensor* t) { return align_up((uint64_t)t->n_row_groups * 4, 256); }

// one u32 arrival ticket per row group, then the partial sums
uint64_t workspace_bytes(const ecw_tensor* t, int batch) {
  const uint64_t p = partial_bytes(t, batch);
  return p ? ticket_bytes(t) + p : 0;
}

}  // namespace ecw

static bool add_ok(uint64_t a, uint64_t b, uint64_t* r) {
  *r = a + b;
  return *r >= a;
}

extern "C" ecw_status dec_prepare(const void* host_blob, size_t blob_bytes, const void* device_blob,
                                  ecw_tensor* out) {
  clear_error();
  if (!host_blob || !out) return fail(ECW_E_INVALID_ARG, "NULL blob or output");
  if (device_blob && (reinterpret_cast<uintptr_t>(device_blob) % 256))
    return fail(ECW_E_INVALID_ARG, "device blob must be 256-byte aligned");
  if (blob_bytes < kHeaderBytes) return fail(ECW_E_CORRUPT, "blob shorter than its header");
  const uint8_t* b = static_cast<const uint8_t*>(host_blob);
  BlobHeader h;
  std::memcpy(&h, b, sizeof(h));
  if (h.magic != kMagic) return fail(ECW_E_CORRUPT, "bad magic");
  if (h.version != kVersion) return fail(ECW_E_UNSUPPORTED, "unknown format version");
  if (h.header_bytes != kHeaderBytes || h.n_sections != kNumSections)
    return fail(ECW_E_CORRUPT, "bad header size or section count");
  if (h.total_bytes != blob_bytes) return fail(ECW_E_CORRUPT, "blob size does not match header");
  ecw_coding c{h.payload, h.rows, h.cols, h.weights_per_symbol, h.code_bits,
               h.log2_m, h.tile_rows, h.tile_cols, h.recon_dtype, h.stored_tuples};
  ecw_status st = check_coding(&c);
  if (st != ECW_OK) return fail(st == ECW_E_UNSUPPORTED ? ECW_E_UNSUPPORTED : ECW_E_CORRUPT,
                                std::string("coding: ") + ecw_last_error());
  Geometry g = geometry_of(c);
  if (h.n_tables != g.n_tables || h.n_row_groups != g.n_rg || h.n_slices != g.n_sl ||
      h.n_tiles != g.n_tiles || h.steps_full != g.s_full || h.steps_last != g.s_last ||
      h.lut_entry_bytes != 8)
    return fail(ECW_E_CORRUPT, "tile geometry does not match the coding");
  const uint32_t M = 1u << c.log2_m;
  const bool bf16 = c.payload == ECW_P_BF16_EXP;
  const bool pairs = bf16 && c.weights_per_symbol == 2;
  const bool quads = quad_coding(c.payload, c.code_bits, c.weights_per_symbol);
  const bool escapes = pairs || quads;
  const uint32_t kw = bf16 ? c.weights_per_symbol : 1;
  // sections: aligned, in bounds, in order, non-overlapping, exact sizes
  uint64_t raw_b = 0;
  if (bf16)
    for (uint32_t sl = 0; sl < g.n_sl; ++sl)
      raw_b += raw_group_count((sl + 1 == g.n_sl ? g.s_last : g.s_full) * kw) * 1024ull * g.n_rg;
  const uint64_t want[kNumSections] = {
      (uint64_t)g.n_tables * sizeof(TableRecord) + (pairs ? kPairDigits : 0) + (quads ? 4ull * c.stored_tuples : 0),
      (uint64_t)g.n_tables * M * 8,
      (uint64_t)g.n_tiles * 256, ((uint64_t)g.n_tiles + 1) * 4, 0, raw_b,
      bf16 ? 0 : (uint64_t)c.rows * 2};
  uint64_t prev_end = kHeaderBytes;
  for (int s = 0; s < (int)kNumSections; ++s) {
    const SectionRef& r = h.sec[s];
    uint64_t end;
    if (r.offset % kSectionAlign) return fail(ECW_E_CORRUPT, "section not 256-byte aligned");
    if (!add_ok(r.offset, r.bytes, &end) || end > blob_bytes)
      return fail(ECW_E_CORRUPT, "section out of bounds");
    if (r.offset < prev_end) return fail(ECW_E_CORRUPT, "sections overlap or out of order");
    if (s != kSecWords && r.bytes != want[s]) return fail(ECW_E_CORRUPT, "section has the wrong size");
    prev_end = end;
  }
  // tables
  uint8_t pair_values[kPairDigits] = {0};
  if (pairs) {
    std::memcpy(pair_values, b + h.sec[kSecTables].offset + g.n_tables * sizeof(TableRecord), kPairDigits);
    if (pair_values[0] != 0) return fail(ECW_E_CORRUPT, "BF16 pairs: digit 0 is not exponent 0");
  }
  std::vector<uint32_t> cum((size_t)g.n_tables * 256);
  std::vector<TableRecord> recs(g.n_tables);
  if (quads) {
    // stored tuples: n of them, ascending, the zero tuple among them, the rest of
    // both arrays zero; frequencies summing to M; decode entries as they define
    TableRecord rec;
    std::memcpy(&rec, b + h.sec[kSecTables].offset, sizeof(TableRecord));
    const uint32_t T = c.stored_tuples, n = rec.alphabet;
    if (n < 1 || n > T) return fail(ECW_E_CORRUPT, "INT quads: stored tuple count out of range");
    for (uint32_t s = 0; s < 256; ++s)
      if (rec.freq[s]) return fail(ECW_E_CORRUPT, "INT quads: the 256-symbol frequencies must be zero");
    std::vector<uint16_t> tup(T), fq(T);
    std::memcpy(tup.data(), b + h.sec[kSecTables].offset + sizeof(TableRecord), 2ull * T);
    std::memcpy(fq.data(), b + h.sec[kSecTables].offset + sizeof(TableRecord) + 2ull * T, 2ull * T);
    bool zero = false;
    uint64_t sum = 0;
    for (uint32_t i = 0; i < T; ++i) {
      if (i >= n) {
        if (tup[i] || fq[i]) return fail(ECW_E_CORRUPT, "INT quads: entries past the stored tuples must be zero");
        continue;
      }
      if (i && tup[i] <= tup[i - 1]) return fail(ECW_E_CORRUPT, "INT quads: stored tuples not ascending");
      zero |= tup[i] == kQuadZero;
      sum += fq[i];
    }
    if (!zero) return fail(ECW_E_CORRUPT, "INT quads: the zero tuple is not stored");
    if (sum != M && !(sum == 0 && g.n_tiles == 0)) return fail(ECW_E_CORRUPT, "tuple frequencies do not sum to M");
    const uint32_t* lut = reinterpret_cast<const uint32_t*>(b + h.sec[kSecLut].offset);
    if (sum == M) {
      uint32_t slot = 0;
      for (uint32_t s = 0; s < n; ++s)
        for (uint32_t i = 0; i < fq[s]; ++i, ++slot) {
          uint32_t lo, hi;
          quad_entry(fq[s], i, tup[s], &lo, &hi);
          if (lut[2 * slot] != lo || lut[2 * slot + 1] != hi)
            return fail(ECW_E_CORRUPT, "decode table does not match the frequencies");
        }
    }
  }
  for (uint32_t k = 0; k < g.n_tables && !quads; ++k) {
    std::memcpy(&recs[k], b + h.sec[kSecTables].offset + k * sizeof(TableRecord), sizeof(TableRecord));
    const TableRecord& rec = recs[k];
    if (rec.alphabet > 256) return fail(ECW_E_CORRUPT, "alphabet > 256");
    uint64_t sum = 0;
    for (uint32_t s = 0; s < 256; ++s) {
      if (s >= rec.alphabet && rec.freq[s]) return fail(ECW_E_CORRUPT, "frequency beyond alphabet");
      cum[k * 256 + s] = (uint32_t)sum;
      sum += rec.freq[s];
    }
    const bool may_be_empty = g.n_tiles == 0 || c.payload == ECW_P_E8_LATTICE;
    if (sum != M && !(sum == 0 && may_be_empty)) return fail(ECW_E_CORRUPT, "table frequencies do not sum to M");
    // decode entries must be the ones the frequencies define
    const uint32_t* lut = reinterpret_cast<const uint32_t*>(b + h.sec[kSecLut].offset) + (size_t)k * M * 2;
    if (sum == M) {
      uint32_t slot = 0;
      for (uint32_t s = 0; s < 256; ++s) {
        uint32_t a8, h16;
        entry_payload(c.payload, c.code_bits, c.weights_per_symbol, rec.value_offset, pair_values, s, &a8, &h16);
        for (uint32_t i = 0; i < rec.freq[s]; ++i, ++slot)
          if (lut[2 * slot] != (rec.freq[s] | (a8 << 24)) || lut[2 * slot + 1] != (i | (h16 << 16)))
            return fail(ECW_E_CORRUPT, "decode table does not match the frequencies");
      }
    }
  }
  // tile meta
  const uint32_t* states = reinterpret_cast<const uint32_t*>(b + h.sec[kSecStates].offset);
  const uint32_t* offs = reinterpret_cast<const uint32_t*>(b + h.sec[kSecOffsets].offset);
  if (offs[0] != 0) return fail(ECW_E_CORRUPT, "first tile offset is not 0");
  for (uint32_t ti = 0; ti < g.n_tiles; ++ti) {
    if (offs[ti + 1] < offs[ti]) return fail(ECW_E_CORRUPT, "tile offsets not monotone");
    const uint32_t rg = ti / g.n_sl, sl = ti % g.n_sl;
    const uint32_t S = (sl + 1 == g.n_sl) ? g.s_last : g.s_full;
    const uint32_t act = std::min<uint32_t>(64, c.rows - rg * 64);
    const uint64_t nwt = (uint64_t)offs[ti + 1] - offs[ti];
    // at most one ANS word per symbol (escapes: plus the lane mask and two words per
    // escaped weight)
    const uint64_t cap = (uint64_t)act * S +
                         (escapes ? kEscMaskWords + 2ull * act * S * c.weights_per_symbol : 0);
    if (nwt > cap) return fail(ECW_E_CORRUPT, "tile holds more words than symbols");
    if (escapes && nwt < kEscMaskWords) return fail(ECW_E_CORRUPT, "tile has no correction stream");
    for (uint32_t l = 0; l < 64; ++l) {
      const uint32_t x = states[(size_t)ti * 64 + l];
      if (l < act ? x < kStateL : x != kStateL)
        return fail(ECW_E_CORRUPT, "tile start state outside [2^16, 2^32)");
    }
  }
  const uint64_t n_words = offs[g.n_tiles];
  if (h.sec[kSecWords].bytes != n_words * 2 + kWordPad)
    return fail(ECW_E_CORRUPT, "word section size does not match the offsets");

  std::memset(out, 0, sizeof(*out));
  out->coding = c;
  out->n_tables = g.n_tables;
  out->n_row_groups = g.n_rg;
  out->n_slices = g.n_sl;
  out->n_tiles = g.n_tiles;
  out->steps_full = g.s_full;
  out->steps_last = g.s_last;
  out->lut_entry_bytes = 8;
  out->blob_bytes = blob_bytes;
  out->bytes_words = n_words * 2;
  out->bytes_raw = raw_b;
  out->bytes_tile_meta = want[kSecStates] + want[kSecOffsets];
  out->bytes_tables = want[kSecTables] + want[kSecLut];
  out->bytes_scales = want[kSecScales];
  out->device_blob = device_blob;
  out->off_tables = h.sec[kSecTables].offset;
  out->off_lut = h.sec[kSecLut].offset;
  out->off_states = h.sec[kSecStates].offset;
  out->off_offsets = h.sec[kSecOffsets].offset;
  out->off_words = h.sec[kSecWords].offset;
  out->off_raw = h.sec[kSecRaw].offset;
  out->off_scales = h.sec[kSecScales].offset;
  default_launch(out);
  return ECW_OK;
}

extern "C" ecw_status dec_gemv_workspace_size(const ecw_tensor* t, int batch, size_t* bytes) {
  clear_error();
  if (!t || !bytes) return fail(ECW_E_INVALID_ARG, "NULL argument");
  if (batch < 1 || batch > 4) return fail(ECW_E_INVALID_ARG, "batch must be 1..4");
  if (t->waves_per_block < 1 || t->waves_per_block > 16 || t->tiles_per_wave < 1)
    return fail(ECW_E_INVALID_ARG, "launch shape out of range");
  *bytes = (size_t)workspace_bytes(t, batch);
  return ECW_OK;
}
