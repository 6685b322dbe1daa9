// Stacks larger than HBM: a device expert-slot cache with LRU replacement,
// the per-layer split of its misses between copies over PCIe and the host
// CPU, and the host expert FFN that serves the misses kept on the CPU.
//
// "DeepSeek-V4.1-Flash served three ways on 4xL20", section 3C (the
// FreeToken engine: every expert in a pinned host store, a device slot cache;
// a miss is copied to the device or computed on the CPU, and the share copied
// is set from the measured bandwidths of the two channels) and section 5 (the
// balance stated as f / (1 - f) = effective PCIe rate / effective CPU rate);
// "Model task radar 2026-11-03: when the accelerator flips", section 6 (the
// first-order form q* ~ m * B_P / B_H); "[Strata] DeepSeek V4.1 Flash on a
// single 4090", section 5.2 (a device LRU of the hottest experts in front of
// a pinned host arena).  Host code only.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "../../include/moe.h"
#include "host_common.h"

struct moe_slot_cache {
  int32_t L = 0, E = 0, S = 0;
  std::vector<int32_t> slot_of;     // [L * E]: the slot holding (layer, expert), or -1
  std::vector<int64_t> owner;       // [S]: the (layer * E + expert) a slot holds, or -1
  std::vector<uint64_t> last_use;   // [S]: the plan step that last used the slot (0: never)
  uint64_t clock = 0;               // plan steps so far
};

namespace {

struct Miss {
  int32_t expert;
  int32_t rows;   // pairs of the step that chose it
};

// a slot for a copy: a free one (lowest index) first, else the least recently
// used one (lowest index on ties) that this step does not already use; -1 if
// every slot is in use by this step
int32_t victim(const moe_slot_cache& c) {
  int32_t best = -1;
  for (int32_t s = 0; s < c.S; ++s) {
    if (c.owner[s] < 0) return s;
    if (c.last_use[s] == c.clock) continue;
    if (best < 0 || c.last_use[s] < c.last_use[best]) best = s;
  }
  return best;
}

}  // namespace

extern "C" int moe_cache_create(int32_t n_layers, int32_t n_experts, int32_t n_slots, moe_slot_cache** out) {
  if (!out) return MOE_EINVAL;
  *out = nullptr;
  if (n_layers <= 0 || n_experts <= 0 || n_slots <= 0) return MOE_EINVAL;
  auto* c = new moe_slot_cache;
  c->L = n_layers;
  c->E = n_experts;
  c->S = n_slots;
  c->slot_of.assign(static_cast<size_t>(n_layers) * n_experts, -1);
  c->owner.assign(static_cast<size_t>(n_slots), -1);
  c->last_use.assign(static_cast<size_t>(n_slots), 0);
  *out = c;
  return MOE_OK;
}

extern "C" void moe_cache_destroy(moe_slot_cache* c) { delete c; }

extern "C" int moe_cache_plan(moe_slot_cache* c, int32_t layer, int32_t rows, int32_t top_k, const int32_t* idx,
                              double copy_share, int32_t* slot_of, int32_t* copy_expert, int32_t* copy_slot,
                              int32_t* n_copy, int32_t* cpu_expert, int32_t* n_cpu, int32_t* idx_gpu) {
  if (!c || !idx || !slot_of || !copy_expert || !copy_slot || !n_copy || !cpu_expert || !n_cpu || !idx_gpu)
    return MOE_EINVAL;
  if (layer < 0 || layer >= c->L || rows < 0 || top_k <= 0 || !(copy_share >= 0.0 && copy_share <= 1.0))
    return MOE_EINVAL;
  const int32_t n = rows * top_k;
  for (int32_t i = 0; i < n; ++i)
    if (idx[i] < 0 || idx[i] >= c->E) return MOE_EINVAL;
  ++c->clock;
  const size_t base = static_cast<size_t>(layer) * c->E;
  // the step's distinct experts in ascending id, with their pair counts
  std::vector<int32_t> cnt(static_cast<size_t>(c->E), 0);
  for (int32_t i = 0; i < n; ++i) ++cnt[static_cast<size_t>(idx[i])];
  std::vector<Miss> misses;
  for (int32_t e = 0; e < c->E; ++e) {
    if (!cnt[static_cast<size_t>(e)]) continue;
    const int32_t s = c->slot_of[base + e];
    if (s >= 0) c->last_use[s] = c->clock;   // hit
    else misses.push_back({e, cnt[static_cast<size_t>(e)]});
  }
  // q of the m misses are copied: with f = copy_share the copies take time
  // proportional to q (1 - f) and the CPU's experts (m - q) f, so q is the
  // whole number next to m f (below or above) with the smaller larger time,
  // the larger q on a tie.  The copied misses are those used by the most
  // pairs (then the lower id), since each saves the CPU the most work.
  const int32_t m = static_cast<int32_t>(misses.size());
  const double f = copy_share;
  const double mf = static_cast<double>(m) * f;
  const int32_t lo = std::min(m, std::max(0, static_cast<int32_t>(std::floor(mf))));
  const int32_t hi = std::min(m, lo + 1);
  auto cost = [&](int32_t qq) {
    return std::max(static_cast<double>(qq) * (1.0 - f), static_cast<double>(m - qq) * f);
  };
  const int32_t q = cost(hi) <= cost(lo) ? hi : lo;
  std::stable_sort(misses.begin(), misses.end(),
                   [](const Miss& a, const Miss& b) { return a.rows > b.rows; });
  std::vector<uint8_t> on_cpu(static_cast<size_t>(c->E), 0);
  int32_t nc = 0, nu = 0;
  for (int32_t j = 0; j < m; ++j) {
    const int32_t e = misses[static_cast<size_t>(j)].expert;
    const int32_t s = j < q ? victim(*c) : -1;
    if (s < 0) {   // not copied: too few slots, or beyond the copy share
      on_cpu[static_cast<size_t>(e)] = 1;
      cpu_expert[nu++] = e;
      continue;
    }
    if (c->owner[s] >= 0) c->slot_of[static_cast<size_t>(c->owner[s])] = -1;   // evict
    c->owner[s] = static_cast<int64_t>(base) + e;
    c->slot_of[base + e] = s;
    c->last_use[s] = c->clock;
    copy_expert[nc] = e;
    copy_slot[nc] = s;
    ++nc;
  }
  std::sort(cpu_expert, cpu_expert + nu);
  *n_copy = nc;
  *n_cpu = nu;
  for (int32_t i = 0; i < n; ++i) idx_gpu[i] = on_cpu[static_cast<size_t>(idx[i])] ? -1 : idx[i];
  for (int32_t e = 0; e < c->E; ++e) slot_of[e] = c->slot_of[base + e];
  return MOE_OK;
}

extern "C" double moe_copy_share(double pcie_bytes_per_s, double cpu_bytes_per_s) {
  if (!(pcie_bytes_per_s >= 0.0) || !(cpu_bytes_per_s >= 0.0)) return 0.0;
  const double t = pcie_bytes_per_s + cpu_bytes_per_s;
  return t > 0.0 ? pcie_bytes_per_s / t : 0.0;
}

namespace {

inline double bf16_to_f64(uint16_t b) {
  const uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return static_cast<double>(f);
}

// rows [n0, n1) of a packed [N x K] matrix times every column of X [R x K]
// (fp64): out[r * ldo + n] = sum_k W[n, k] X[r, k].  Decodes kRowBlock rows
// at a time into a local buffer; false if a code is invalid.
bool gemv_rows(int fmt, const uint8_t* w, int64_t N, int64_t K, const double* X, int R, double* out, int64_t ldo,
               int64_t n0, int64_t n1) {
  constexpr int64_t kRowBlock = 8;
  std::vector<float> buf(static_cast<size_t>(kRowBlock * K));
  for (int64_t a = n0; a < n1; a += kRowBlock) {
    const int64_t b = std::min(n1, a + kRowBlock);
    if (!moe::unpack_rows(fmt, w, N, K, buf.data(), a, b)) return false;
    for (int64_t n = a; n < b; ++n) {
      const float* wr = buf.data() + (n - a) * K;
      for (int r = 0; r < R; ++r) {
        const double* xr = X + static_cast<size_t>(r) * K;
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) s += static_cast<double>(wr[k]) * xr[k];
        out[static_cast<size_t>(r) * ldo + n] = s;
      }
    }
  }
  return true;
}

template <class F>
bool parallel_ok(int64_t n, int nthreads, F&& body) {
  int t = nthreads > 0 ? nthreads : static_cast<int>(std::thread::hardware_concurrency());
  t = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(t, n)));
  std::vector<uint8_t> ok(static_cast<size_t>(t), 1);
  std::vector<std::thread> pool;
  const int64_t per = (n + t - 1) / t;
  for (int i = 0; i < t; ++i) {
    const int64_t a = i * per, b = std::min(n, a + per);
    if (a >= b) continue;
    pool.emplace_back([&, i, a, b] { ok[static_cast<size_t>(i)] = body(a, b) ? 1 : 0; });
  }
  for (auto& th : pool) th.join();
  for (uint8_t v : ok)
    if (!v) return false;
  return true;
}

}  // namespace

extern "C" int moe_cpu_expert_ffn(const moe_dims* dims, int32_t fmt, const void* gate, const void* up,
                                  const void* down, const void* x_bf16, int32_t n_rows, const int32_t* row_ids,
                                  const float* row_w, float* y, int32_t n_threads) {
  if (!dims || !gate || !up || !down || !x_bf16 || !y || (n_rows > 0 && (!row_ids || !row_w))) return MOE_EINVAL;
  if (n_rows < 0) return MOE_EINVAL;
  if (moe::format_info(fmt).block == 0) return MOE_EFORMAT;
  const int64_t H = dims->hidden, I = dims->inter;
  if (H <= 0 || I <= 0 || moe::blocks_per_row(fmt, H) < 0 || moe::blocks_per_row(fmt, I) < 0) return MOE_ESHAPE;
  if (n_rows == 0) return MOE_OK;
  const uint16_t* xb = static_cast<const uint16_t*>(x_bf16);
  std::vector<double> X(static_cast<size_t>(n_rows) * H);
  for (int r = 0; r < n_rows; ++r) {
    if (row_ids[r] < 0) return MOE_EINVAL;
    for (int64_t h = 0; h < H; ++h)
      X[static_cast<size_t>(r) * H + h] = bf16_to_f64(xb[static_cast<size_t>(row_ids[r]) * H + h]);
  }
  // g = Wg x, v = Wu x, h = silu(g) * v, o = Wd h: all sums in fp64
  std::vector<double> G(static_cast<size_t>(n_rows) * I), V(static_cast<size_t>(n_rows) * I);
  const auto* wg = static_cast<const uint8_t*>(gate);
  const auto* wu = static_cast<const uint8_t*>(up);
  const auto* wd = static_cast<const uint8_t*>(down);
  if (!parallel_ok(I, n_threads, [&](int64_t a, int64_t b) {
        return gemv_rows(fmt, wg, I, H, X.data(), n_rows, G.data(), I, a, b) &&
               gemv_rows(fmt, wu, I, H, X.data(), n_rows, V.data(), I, a, b);
      }))
    return MOE_ECODE;
  for (size_t i = 0; i < G.size(); ++i) G[i] = G[i] / (1.0 + std::exp(-G[i])) * V[i];
  std::vector<double> O(static_cast<size_t>(n_rows) * H);
  if (!parallel_ok(H, n_threads, [&](int64_t a, int64_t b) {
        return gemv_rows(fmt, wd, H, I, G.data(), n_rows, O.data(), H, a, b);
      }))
    return MOE_ECODE;
  for (int r = 0; r < n_rows; ++r) {
    float* yr = y + static_cast<size_t>(row_ids[r]) * H;
    const double wr = static_cast<double>(row_w[r]);
    for (int64_t h = 0; h < H; ++h) yr[h] = static_cast<float>(static_cast<double>(yr[h]) + wr * O[static_cast<size_t>(r) * H + h]);
  }
  return MOE_OK;
}
