// Host entry of the many-row (prefill) path: MXFP4 experts on the scaled
// matrix cores, activations in MXFP8.
#pragma once
#include <cstddef>
#include <cstdint>

#include "../../include/moe.h"

namespace moe {
namespace pf {

size_t workspace_bytes(const moe_dims& d, int rows);
int run(const moe_dims* d, const void* x, int rows, const int32_t* idx, const float* wts,
        const void* weights, const moe_expert_ref* experts, const moe_expert_ref* shared, float* y,
        void* ws, size_t ws_bytes, void* stream);
int quant(const void* x, int rows, int K, void* codes, void* scales, void* stream);

}  // namespace pf
}  // namespace moe
