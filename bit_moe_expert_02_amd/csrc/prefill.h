// Host entries of the many-row path: MXFP4 experts on the scaled matrix
// cores (activations in MXFP8), every other expert through the decode tiles.
#pragma once
#include <cstddef>
#include <cstdint>

#include "../../include/moe.h"
#include "layout.h"

namespace moe {
namespace pf {

int run(const moe_dims* d, const void* x, int rows, const int32_t* idx, const float* wts,
        const void* weights, const moe_expert_ref* experts, const moe_expert_ref* shared, float* y,
        void* ws, size_t ws_bytes, void* stream);
int quant(const void* x, int rows, int K, void* codes, void* scales, void* stream);

}  // namespace pf

namespace gen {

// The generic part of a many-row call: device buffers from the workspace and
// the call's arguments (layout.h, ManyRowLayout).
struct Launch {
  const void* x;
  const int32_t* idx;
  const float* wts;
  const void* weights;
  const moe_expert_ref* experts;
  const moe_expert_ref* shared;
  const int32_t* cnt;
  const int32_t* list;
  lay::GenEntry* gen;
  int32_t* gen_n;
  int32_t* map_gu;
  int32_t* map_dn;
  float* h32;
  float* part;
  int rows, top_k, n_experts, mfma;
  int max_gen, max_items_gu, max_items_dn;
};

// Plans the generic entries (after the pair lists exist) and runs their
// gate/up and down items; asynchronous on `stream`.
int launch(const moe_dims* d, const Launch& g, void* stream);

}  // namespace gen
}  // namespace moe
