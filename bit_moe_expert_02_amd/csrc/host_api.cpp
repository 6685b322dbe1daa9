// Host validation of the C ABI: status strings, dims checks, workspace sizes
// and the expert-table check.  Plain C++ with no HIP calls, so it builds with
// any host compiler (the sanitizer build of the host code includes it).

#include "host_api.h"

#include "host_common.h"

namespace moe {

namespace {
constexpr uint32_t kKnownFlags = MOE_ACT_MXFP8;

int check_common(const moe_dims* d) {
  if (!d) return MOE_EINVAL;
  if (d->flags & ~kKnownFlags) return MOE_EINVAL;
  if (!lay::shape_class(*d)) return MOE_ESHAPE;
  if (d->top_k < 1 || d->top_k > MOE_MAX_TOP_K || d->n_experts < d->top_k ||
      d->n_experts > lay::kMaxExperts)
    return MOE_ESHAPE;
  return MOE_OK;
}
}  // namespace

int check_dims(const moe_dims* d, int rows) {
  if (int st = check_common(d)) return st;
  if (rows < 0) return MOE_EINVAL;
  if (rows > MOE_MAX_DECODE_ROWS || rows * d->top_k > lay::kMaxSlots) return MOE_ESHAPE;
  return MOE_OK;
}

int check_many_row_dims(const moe_dims* d, int rows) {
  if (int st = check_common(d)) return st;
  if (rows <= MOE_MAX_DECODE_ROWS || rows > MOE_MAX_PREFILL_ROWS) return MOE_ESHAPE;
  return MOE_OK;
}

}  // namespace moe

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_ESHAPE: return "unsupported shape";
    case MOE_EFORMAT: return "unknown weight format";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EDEVICE: return "HIP launch or runtime error";
    case MOE_ECODE: return "invalid packed code";
    case MOE_ETIMEOUT: return "a hand-off wait of the fused layer gave up";
    default: return "unknown status";
  }
}

size_t moe_workspace_bytes(const moe_dims* dims, int32_t rows) {
  if (rows > MOE_MAX_DECODE_ROWS) {
    if (moe::check_many_row_dims(dims, rows)) return 0;
    return moe::lay::many_row_layout(*dims, rows).total;
  }
  if (moe::check_dims(dims, rows < 1 ? 1 : rows)) return 0;
  return moe::lay::decode_layout(*dims, rows < 1 ? 1 : rows).total;
}

int moe_check_experts(const moe_dims* dims, const moe_expert_ref* table, int32_t count,
                      size_t weights_bytes) {
  if (!dims || !table || count < 0) return MOE_EINVAL;
  if (!moe::lay::shape_class(*dims)) return MOE_ESHAPE;
  for (int i = 0; i < count; ++i) {
    const moe_expert_ref& r = table[i];
    if (moe::format_info(static_cast<int>(r.fmt)).block == 0) return MOE_EFORMAT;
    if (r.reserved != 0) return MOE_EINVAL;
    const size_t gu = moe::packed_bytes(static_cast<int>(r.fmt), dims->inter, dims->hidden);
    const size_t dn = moe::packed_bytes(static_cast<int>(r.fmt), dims->hidden, dims->inter);
    if (!gu || !dn) return MOE_ESHAPE;
    const uint64_t offs[3] = {r.gate, r.up, r.down};
    const size_t sizes[3] = {gu, gu, dn};
    for (int m = 0; m < 3; ++m) {
      if (offs[m] % 16) return MOE_EINVAL;
      if (offs[m] > weights_bytes || sizes[m] > weights_bytes - offs[m]) return MOE_EINVAL;
    }
  }
  return MOE_OK;
}

}  // extern "C"
