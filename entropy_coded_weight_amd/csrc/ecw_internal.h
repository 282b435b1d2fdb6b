// Internal declarations shared by the host encoder / validator and the kernel
// launchers.  Not part of the public ABI.
#pragma once
#include <stdint.h>

#include <string>

#include "../../include/ecw.h"
#include "ecw_format.h"

namespace ecw {

// thread-local error text behind ecw_last_error()
ecw_status fail(ecw_status s, const std::string& msg);
void clear_error();

// coding checks common to encoder, validator and launchers
ecw_status check_coding(const ecw_coding* c);

struct Geometry {
  uint32_t n_tables, n_rg, n_sl, n_tiles, s_full, s_last, syms_per_row;
};
Geometry geometry_of(const ecw_coding& c);

// launch shape helpers
void default_launch(ecw_tensor* t);
// LDS bytes of one block of the fused kernel (or, with mat, the decode-only hook)
// for W waves of R tiles at batch capacity B (1 or 4); xbf: bf16 activations.
uint64_t launch_lds_bytes(const ecw_tensor* t, uint32_t W, uint32_t R, int B, bool mat, bool xbf);
uint32_t slice_groups(const ecw_tensor* t);
uint64_t workspace_bytes(const ecw_tensor* t, int batch);
// a tensor's workspace: arrival tickets (one per row group), then per-block partial sums
uint64_t ticket_bytes(const ecw_tensor* t);
uint64_t partial_bytes(const ecw_tensor* t, int batch);

}  // namespace ecw
