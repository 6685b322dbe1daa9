// Host-side checks of libmoe's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitized.py together with
// the packer (pack.cpp) and the host validation (host_api.cpp) -- no HIP.
//
//   * packer: pack -> unpack -> pack gives the same bytes (every format but
//     Q3) over a range of shapes (ragged row counts, the ternary padding), unpack
//     rejects invalid codes, every argument error returns its status;
//   * expert tables: moe_check_experts' format, alignment and bounds checks;
//   * workspaces: every region of every row count lies past the tagged area
//     of the fused launch, inside moe_workspace_bytes, without overlaps, and
//     the tagged area is the same for every row count.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <utility>
#include <vector>

#include "../bit_moe_expert_02_amd/csrc/host_api.h"
#include "../bit_moe_expert_02_amd/csrc/layout.h"
#include "../include/moe.h"

namespace {

int failures = 0;

void check(bool ok, const std::string& what) {
  if (!ok) {
    std::fprintf(stderr, "FAIL: %s\n", what.c_str());
    ++failures;
  }
}

const int kFormats[] = {MOE_FMT_TERN160, MOE_FMT_Q2_0, MOE_FMT_Q3, MOE_FMT_MXFP4, MOE_FMT_Q8};

void packer_round_trips() {
  std::mt19937 rng(7);
  std::normal_distribution<float> nd(0.0f, 0.02f);
  const std::pair<int, int> shapes[] = {{1, 256}, {3, 512}, {17, 2304}, {64, 5120 / 4}, {5, 160}, {2, 480}};
  for (int fmt : kFormats) {
    for (auto [n, k] : shapes) {
      const size_t nb = moe_packed_bytes(fmt, n, k);
      if (nb == 0) continue;   // K not a block multiple for this format
      std::vector<float> w(static_cast<size_t>(n) * k), back(w.size());
      for (float& v : w) v = nd(rng);
      w[0] = 0.0f;             // a zero and a large outlier per matrix
      w[w.size() / 2] = 3.0f;
      std::vector<uint8_t> p1(nb), p2(nb);
      check(moe_pack(fmt, w.data(), n, k, p1.data(), nb, 3) == MOE_OK, "pack");
      check(moe_unpack(fmt, p1.data(), nb, n, k, back.data(), 2) == MOE_OK, "unpack");
      check(moe_pack(fmt, back.data(), n, k, p2.data(), nb, 1) == MOE_OK, "repack");
      // RTN is a projection for every format but Q3, whose sub-blocks with a
      // scale that rounds to a small integer can requantise differently
      if (fmt != MOE_FMT_Q3)
        check(p1 == p2, "pack(unpack(pack(w))) == pack(w), fmt " + std::to_string(fmt) + " " +
                            std::to_string(n) + "x" + std::to_string(k));
      // argument errors
      check(moe_pack(fmt, nullptr, n, k, p1.data(), nb, 1) == MOE_EINVAL, "null w");
      check(moe_pack(fmt, w.data(), n, k, p1.data(), nb - 1, 1) == MOE_EINVAL, "short dst");
      check(moe_unpack(fmt, p1.data(), nb - 1, n, k, back.data(), 1) == MOE_EINVAL, "short src");
      check(moe_pack(fmt, w.data(), 0, k, p1.data(), nb, 1) == MOE_EINVAL, "n = 0");
    }
  }
  check(moe_pack(9, nullptr, 1, 64, nullptr, 0, 1) == MOE_EFORMAT, "unknown format");
  check(moe_packed_bytes(MOE_FMT_Q2_0, 4, 100) == 0, "K not a block multiple");
  check(moe_packed_bytes(MOE_FMT_TERN160, 4, 100) == 4 * 34, "ternary pads");
  // invalid codes: a ternary byte above 242, an e8m0 scale of 255
  {
    const size_t nb = moe_packed_bytes(MOE_FMT_TERN160, 1, 160);
    std::vector<uint8_t> p(nb, 121);   // all-zero trits
    std::vector<float> out(160);
    check(moe_unpack(MOE_FMT_TERN160, p.data(), nb, 1, 160, out.data(), 1) == MOE_OK, "valid ternary");
    p[5] = 243;
    check(moe_unpack(MOE_FMT_TERN160, p.data(), nb, 1, 160, out.data(), 1) == MOE_ECODE, "ternary 243");
  }
  {
    const size_t nb = moe_packed_bytes(MOE_FMT_MXFP4, 2, 64);
    std::vector<uint8_t> p(nb, 0);
    std::vector<float> out(128);
    p[nb - 1] = 255;
    check(moe_unpack(MOE_FMT_MXFP4, p.data(), nb, 2, 64, out.data(), 1) == MOE_ECODE, "e8m0 255");
  }
}

void expert_tables() {
  const moe_dims d{5120, 2304, 384, 6, 0};
  const size_t gu = moe_packed_bytes(MOE_FMT_Q2_0, 2304, 5120), dn = moe_packed_bytes(MOE_FMT_Q2_0, 5120, 2304);
  const size_t total = 2 * gu + dn;
  moe_expert_ref r{MOE_FMT_Q2_0, 0, 0, gu, 2 * gu};
  check(moe_check_experts(&d, &r, 1, total) == MOE_OK, "good table");
  check(moe_check_experts(&d, &r, 1, total - 1) == MOE_EINVAL, "matrix past the buffer");
  moe_expert_ref bad = r;
  bad.up = gu + 8;
  check(moe_check_experts(&d, &bad, 1, total + 64) == MOE_EINVAL, "misaligned offset");
  bad = r;
  bad.fmt = 7;
  check(moe_check_experts(&d, &bad, 1, total) == MOE_EFORMAT, "unknown format");
  bad = r;
  bad.reserved = 1;
  check(moe_check_experts(&d, &bad, 1, total) == MOE_EINVAL, "reserved field");
  bad = r;
  bad.down = ~0ull - 8;   // offset near the top of the address range: no wrap-around
  check(moe_check_experts(&d, &bad, 1, total) == MOE_EINVAL, "huge offset");
  const moe_dims odd{4096, 2304, 384, 6, 0};
  check(moe_check_experts(&odd, &r, 1, total) == MOE_ESHAPE, "unsupported shape");
  check(moe_check_experts(&d, nullptr, 1, total) == MOE_EINVAL, "null table");
}

struct Region {
  size_t a, b;
  const char* name;
};

void check_regions(std::vector<Region> rs, size_t tagged_end, size_t total, const std::string& tag) {
  for (const Region& r : rs) {
    check(r.a >= tagged_end, tag + ": " + r.name + " starts inside the tagged area");
    check(r.b <= total, tag + ": " + r.name + " ends past the workspace");
    check(r.a <= r.b, tag + ": " + r.name + " has negative size");
  }
  for (size_t i = 0; i < rs.size(); ++i)
    for (size_t j = i + 1; j < rs.size(); ++j)
      check(rs[i].b <= rs[j].a || rs[j].b <= rs[i].a,
            tag + ": " + rs[i].name + " overlaps " + rs[j].name);
}

void workspaces() {
  using namespace moe::lay;
  const moe_dims dims_list[] = {{5120, 2304, 384, 6, 0}, {5120, 2304, 128, 3, 0}, {512, 256, 16, 2, 0},
                                {512, 256, 500, 8, 0}, {5120, 2304, 384, 6, MOE_ACT_MXFP8}};
  for (const moe_dims& d : dims_list) {
    const TaggedLayout t = tagged_layout(d);
    const std::string dn = std::to_string(d.hidden) + "/" + std::to_string(d.n_experts) + "/" +
                           std::to_string(d.top_k);
    // the tagged area holds kMaxRows rows of everything the fused launch tags
    const size_t pairs = static_cast<size_t>(kMaxRows) * d.top_k + kMaxRows;
    check(t.lgt >= t.err + 4 && t.selt >= t.lgt + 16ull * kMaxRows * d.n_experts &&
              t.ht >= t.selt + 8ull * kSelRep * kSelRepWords && t.part_t >= t.ht + 8 * pairs * d.inter &&
              t.end >= t.part_t + 8 * pairs * d.hidden,
          dn + ": tagged area sizes");
    for (int rows = 1; rows <= MOE_MAX_DECODE_ROWS; ++rows) {
      if (rows * d.top_k > kMaxSlots) continue;
      const DecodeLayout l = decode_layout(d, rows);
      check(moe_workspace_bytes(&d, rows) == l.total, dn + ": decode workspace size");
      const size_t P = static_cast<size_t>(rows) * d.top_k, PS = P + rows;
      check_regions({{l.logits, l.logits + 8 * rows * static_cast<size_t>(d.n_experts), "logits"},
                     {l.idx, l.idx + 4 * P, "idx"},
                     {l.wts, l.wts + 4 * P, "wts"},
                     {l.slots, l.slots + sizeof(SlotTable), "slots"},
                     {l.order, l.order + 4 * P, "order"},
                     {l.xinv, l.xinv + 4 * kNumFmt * static_cast<size_t>(rows), "xinv"},
                     {l.xrec, l.xrec + static_cast<size_t>(kNumFmt) * rows * l.xrow, "xrec"},
                     {l.h, l.h + 4 * PS * d.inter, "h"},
                     {l.part, l.part + 4 * PS * d.hidden, "part"}},
                    t.end, l.total, dn + " decode rows " + std::to_string(rows));
    }
    for (int rows : {9, 10, 16, 55, 64, 100, 1000, 2048, 4097, 8192}) {
      const ManyRowLayout l = many_row_layout(d, rows);
      check(moe_workspace_bytes(&d, rows) == l.total, dn + ": many-row workspace size");
      const size_t R = rows, P = R * d.top_k, PS = P + R;
      check_regions({{l.xq, l.xq + R * d.hidden, "xq"},
                     {l.xs, l.xs + R * d.hidden / 32, "xs"},
                     {l.cnt, l.cnt + 4 * static_cast<size_t>(d.n_experts), "cnt"},
                     {l.list, l.list + 4 * P, "list"},
                     {l.chunks, l.chunks + sizeof(Chunk) * static_cast<size_t>(l.max_chunks), "chunks"},
                     {l.n_chunks, l.n_chunks + 4, "n_chunks"},
                     {l.gen, l.gen + sizeof(GenEntry) * static_cast<size_t>(l.max_gen), "gen"},
                     {l.n_gen, l.n_gen + 12, "n_gen"},
                     {l.map_gu, l.map_gu + 4 * static_cast<size_t>(l.max_items_gu), "map_gu"},
                     {l.map_dn, l.map_dn + 4 * static_cast<size_t>(l.max_items_dn), "map_dn"},
                     {l.hq, l.hq + 2 * P * d.inter, "hq"},
                     {l.h32, l.h32 + 4 * PS * d.inter, "h32"},
                     {l.part, l.part + 4 * PS * d.hidden, "part"}},
                    t.end, l.total, dn + " many rows " + std::to_string(rows));
      // every expert's entries (ceil(cnt/8) each) and the shared expert's fit
      check(l.max_gen >= static_cast<int>((P + kGenRows - 1) / kGenRows) + d.n_experts, dn + ": entry bound");
      check(l.max_chunks >= static_cast<int>((P + kChunk - 1) / kChunk) + d.n_experts, dn + ": chunk bound");
    }
  }
  // a workspace sized for one use serves every other: the tagged area never moves
  const moe_dims d{5120, 2304, 384, 6, 0};
  check(moe_workspace_bytes(&d, 1) >= tagged_layout(d).end, "decode workspace holds the tagged area");
  check(moe_workspace_bytes(&d, 55) >= tagged_layout(d).end, "many-row workspace holds the tagged area");
}

void allocator() {
  // a random 5-layer, 40-expert instance: guardrails hold, bytes within budget
  const int L = 5, E = 40;
  std::mt19937 rng(3);
  std::uniform_real_distribution<double> u(0.05, 1.0);
  std::vector<double> err(static_cast<size_t>(L) * E * 3), energy(L);
  std::vector<int32_t> tokens(static_cast<size_t>(L) * E);
  for (double& v : err) v = u(rng);
  for (double& v : energy) v = u(rng);
  for (size_t i = 0; i < tokens.size(); ++i) tokens[i] = static_cast<int32_t>(i % 50);
  const uint64_t fb[3] = {7624704, 9953280, 15206400};
  std::vector<uint8_t> fmt(static_cast<size_t>(L) * E);
  double cost = 0.0;
  uint64_t bytes = 0;
  check(moe_allocate_formats(L, E, err.data(), tokens.data(), energy.data(), fb, 0.5, 8, 2, 3, fmt.data(), &cost,
                             &bytes) == MOE_OK, "allocate");
  check(bytes <= static_cast<uint64_t>(L) * E * fb[1], "allocation within budget");
  for (int l = 0; l < L; ++l) {
    int tern = 0;
    for (int e = 0; e < E; ++e) {
      const uint8_t f = fmt[static_cast<size_t>(l) * E + e];
      tern += f == MOE_FMT_TERN160;
      if (tokens[static_cast<size_t>(l) * E + e] < 8) check(f == MOE_FMT_Q2_0, "locked expert stays Q2_0");
    }
    check(tern <= E / 2, "ternary cap");
  }
  const uint64_t bad[3] = {fb[1], fb[0], fb[2]};
  check(moe_allocate_formats(L, E, err.data(), tokens.data(), energy.data(), bad, 0.5, 8, 2, 3, fmt.data(),
                             nullptr, nullptr) == MOE_EINVAL, "unordered sizes");
  check(moe_allocate_formats(0, E, err.data(), tokens.data(), energy.data(), fb, 0.5, 8, 2, 3, fmt.data(),
                             nullptr, nullptr) == MOE_EINVAL, "no layers");
}

void offload() {
  // the slot cache over a random sequence: every selected expert ends on the
  // device or on the CPU, never both; bad input is rejected
  moe_slot_cache* c = nullptr;
  check(moe_cache_create(2, 32, 5, &c) == MOE_OK && c, "cache create");
  std::mt19937 rng(5);
  std::vector<int32_t> idx(16), slot_of(32), ce(16), cs(16), cpu(16), idx_gpu(16);
  for (int step = 0; step < 200; ++step) {
    const int rows = 1 + static_cast<int>(rng() % 4), k = 4;
    for (int i = 0; i < rows * k; ++i) idx[i] = static_cast<int32_t>(rng() % 32);
    int32_t nc = 0, nu = 0;
    const double share = (rng() % 5) / 4.0;
    check(moe_cache_plan(c, step % 2, rows, k, idx.data(), share, slot_of.data(), ce.data(), cs.data(), &nc,
                         cpu.data(), &nu, idx_gpu.data()) == MOE_OK, "plan");
    for (int i = 0; i < rows * k; ++i) {
      bool on_cpu = false;
      for (int j = 0; j < nu; ++j) on_cpu = on_cpu || cpu[j] == idx[i];
      check(on_cpu != (slot_of[idx[i]] >= 0), "device xor cpu");
      check(idx_gpu[i] == (on_cpu ? -1 : idx[i]), "idx_gpu");
    }
  }
  idx[0] = 32;
  int32_t nc = 0, nu = 0;
  check(moe_cache_plan(c, 0, 1, 1, idx.data(), 1.0, slot_of.data(), ce.data(), cs.data(), &nc, cpu.data(), &nu,
                       idx_gpu.data()) == MOE_EINVAL, "id out of range");
  check(moe_cache_plan(c, 2, 1, 1, idx.data(), 1.0, slot_of.data(), ce.data(), cs.data(), &nc, cpu.data(), &nu,
                       idx_gpu.data()) == MOE_EINVAL, "layer out of range");
  moe_cache_destroy(c);
  moe_slot_cache* none = nullptr;
  check(moe_cache_create(1, 8, 0, &none) == MOE_EINVAL && !none, "no slots");
  check(moe_copy_share(3.0, 1.0) == 0.75, "copy share");
  // the host FFN on a small Q2_0 expert, one row
  const moe_dims d{64, 64, 8, 2, 0};
  const size_t nb = moe_packed_bytes(MOE_FMT_Q2_0, 64, 64);
  std::vector<float> w(64 * 64);
  std::normal_distribution<float> nd(0.0f, 0.02f);
  for (float& v : w) v = nd(rng);
  std::vector<uint8_t> m(nb);
  check(moe_pack(MOE_FMT_Q2_0, w.data(), 64, 64, m.data(), nb, 1) == MOE_OK, "pack for ffn");
  std::vector<uint16_t> x(2 * 64, 0x3f80);   // bf16 1.0
  std::vector<float> y(2 * 64, 0.0f);
  const int32_t row = 1;
  const float rw = 0.5f;
  check(moe_cpu_expert_ffn(&d, MOE_FMT_Q2_0, m.data(), m.data(), m.data(), x.data(), 1, &row, &rw, y.data(), 2) ==
            MOE_OK, "cpu ffn");
  bool row0_zero = true;
  for (int i = 0; i < 64; ++i) row0_zero = row0_zero && y[i] == 0.0f;
  check(row0_zero, "cpu ffn leaves other rows");
  check(moe_cpu_expert_ffn(&d, 9, m.data(), m.data(), m.data(), x.data(), 1, &row, &rw, y.data(), 1) == MOE_EFORMAT,
        "cpu ffn format");
}

void dims_checks() {
  const moe_dims good{5120, 2304, 384, 6, 0};
  check(moe::check_dims(&good, 8) == MOE_OK, "8 rows");
  check(moe::check_dims(&good, 9) == MOE_ESHAPE, "9 decode rows");
  check(moe::check_dims(&good, -1) == MOE_EINVAL, "negative rows");
  check(moe::check_dims(nullptr, 1) == MOE_EINVAL, "null dims");
  const moe_dims flags{5120, 2304, 384, 6, 2};
  check(moe::check_dims(&flags, 1) == MOE_EINVAL, "unknown flag");
  check(moe_workspace_bytes(&flags, 1) == 0, "unknown flag: no workspace");
  const moe_dims k9{5120, 2304, 384, 9, 0};
  check(moe::check_dims(&k9, 1) == MOE_ESHAPE, "top_k 9");
  const moe_dims e513{5120, 2304, 513, 6, 0};
  check(moe::check_dims(&e513, 1) == MOE_ESHAPE, "513 experts");
  check(moe::check_many_row_dims(&good, 8192) == MOE_OK, "8192 rows");
  check(moe::check_many_row_dims(&good, 8193) == MOE_ESHAPE, "8193 rows");
  check(moe::check_many_row_dims(&good, 8) == MOE_ESHAPE, "8 rows are decode rows");
  for (int st = 1; st >= -8; --st) check(moe_status_string(st) != nullptr, "status string");
}

}  // namespace

int main() {
  packer_round_trips();
  expert_tables();
  workspaces();
  dims_checks();
  allocator();
  offload();
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("host checks ok\n");
  return 0;
}
