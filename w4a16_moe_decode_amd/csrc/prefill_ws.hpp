// Prefill workspace view (offsets computed on the host by carve_prefill_ws).
#pragma once

#include "common.hpp"

namespace flint {

struct PrefillWs {
  uint16_t* xn;          // [T][H]
  float* logits;         // [T][E]
  int32_t* idx;          // [T][K]
  float* wgt;            // [T][K]
  uint64_t* cmask;       // [C][E] token bitmask per chunk and expert
  int32_t* cbase;        // [C][E] first permuted position of the chunk's pairs of e
  int32_t* counts;       // [E + 1]
  int32_t* offsets;      // [E + 2]
  int32_t* ntiles;       // [1]
  int2* tiles;           // [max_tiles] (group, first row)
  int32_t* perm_tok;     // [T*K]
  float* perm_w;         // [T*K]
  int32_t* pos;          // [T][K]
  uint16_t* h;           // [T*K + T][Imax]
  float* y;              // [T*K + T][H]
  uint16_t* router_f;    // [E*H] the router in the fused routing kernel's fragment order (H 2048, E 256), else null
  int max_tiles;
  int64_t bytes;
};

int prefill_max_tiles(const flint_moe_shape& s, int T);
int64_t prefill_ws_bytes(const flint_moe_shape& s, int T);

}  // namespace flint
