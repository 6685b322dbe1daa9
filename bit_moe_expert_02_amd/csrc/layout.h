// Sizes and plain structs that the host code and the gfx950 kernels share:
// the workspace layout of every entry point, the slot table of the decode
// path and the work lists of the many-row path.  Plain C++ (no HIP), so the
// host validation builds and runs on a CPU alone.
#pragma once
#include <cstddef>
#include <cstdint>

#include "../../include/moe.h"

namespace moe {
namespace lay {

constexpr int kMaxRows = MOE_MAX_DECODE_ROWS;  // rows per decode call
constexpr int kMaxK = MOE_MAX_TOP_K;
constexpr int kMaxSlots = 64;                  // distinct routed experts per decode call (rows * top_k)
constexpr int kNumFmt = 5;                     // format tags 1..5
constexpr int kMaxExperts = 512;               // routed experts a layer may have
constexpr int kThreads = 256;                  // threads of a decode workgroup

// The fused launch publishes the selection as kSelWords tagged words per
// entry (id | fmt << 16, weight bits, then the 32-bit halves of the gate, up
// and down offsets) in kSelRep copies, kSelRepWords apart; word
// kSelEntryWords of a copy is the "every logit is out" flag.
constexpr int kSelWords = 8;
constexpr int kSelRep = 16;
constexpr int kSelEntryWords = kMaxRows * kMaxK * kSelWords;
constexpr int kSelRepWords = kSelEntryWords + 64;

// Rows of the many-row path: pairs of one expert per matrix-core work item,
// and pairs per generic (decode-tile) work entry.
constexpr int kChunk = 64;
constexpr int kGenRows = kMaxRows;

// Bytes of one activation record row of a format for reduction length k:
// units(k) * record bytes per unit, as the decode engines lay them out.
constexpr int rec_row_bytes(int fmt, int k) {
  return fmt == MOE_FMT_Q2_0      ? (k / 64) * 144
         : fmt == MOE_FMT_Q8      ? (k / 32) * 80
         : fmt == MOE_FMT_MXFP4   ? (k / 32) * 80
         : fmt == MOE_FMT_TERN160 ? 2 * ((k + 159) / 160) * 176
         : fmt == MOE_FMT_Q3      ? (k / 64) * 144
                                  : 0;
}
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int max_rec_row(int k) {
  return cmax(cmax(cmax(rec_row_bytes(MOE_FMT_Q2_0, k), rec_row_bytes(MOE_FMT_Q8, k)),
                   cmax(rec_row_bytes(MOE_FMT_MXFP4, k), rec_row_bytes(MOE_FMT_TERN160, k))),
              rec_row_bytes(MOE_FMT_Q3, k));
}

// One entry of the decode slot table: a distinct selected expert (or the
// shared one) and the rows it serves.
struct SlotEntry {
  moe_expert_ref ref;       // format and matrix offsets, copied from the expert table
  int expert;               // routed id, -1 for the shared expert
  int nt;                   // rows served
  int row[kMaxRows];        // token row r
  int pair[kMaxRows];       // h / partial row: r*k + kk (routed) or R*k + r (shared)
  float w[kMaxRows];        // mixing weight (1 for the shared expert)
};

// The work of one decode call: slots [0, n_active) are the distinct routed
// experts in ascending id, slot n_active the shared expert (when there is
// one).  Work item i of the gate/up (down) list is tile i - gu_off[s] of the
// slot s with gu_off[s] <= i < gu_off[s + 1].
struct SlotTable {
  int n_active;
  int n_slots;
  int n_gu, n_dn;
  int gu_off[kMaxSlots + 2];
  int dn_off[kMaxSlots + 2];
  SlotEntry e[kMaxSlots + 1];
};

// Many-row path: a matrix-core work item (at most kChunk pairs of one
// MXFP4 expert) ...
struct Chunk {
  int expert;   // routed id
  int s0;       // first position in the expert-sorted pair list
  int m;        // pairs in this chunk (1 .. kChunk)
};
// ... and a generic work entry: at most kGenRows pairs of one expert run
// through the decode tiles (any format; expert -1 is the shared expert,
// whose pairs are R*k + r).
struct GenEntry {
  int expert;
  int s0;       // first position in the expert-sorted pair list (routed)
                // or first row (shared)
  int m;        // pairs (1 .. kGenRows)
  int gu_off;   // first gate/up item of this entry
  int dn_off;   // first down item of this entry
};

// ---------------------------------------------------------------------------
// Workspace layout.  Every workspace starts with the tagged area of the fused
// decode launch, whose size depends on the dims only (it is laid out for
// kMaxRows rows): the error word, the logits as tagged halves, the
// published selection, h and the partial outputs.  Those words are only ever
// written with a call tag in the upper half, by the fused launch.  Every
// other region of every entry point starts past it, so no untagged store can
// leave a word there that a later fused call would take for its own.
// ---------------------------------------------------------------------------
struct TaggedLayout {
  size_t err, lgt, selt, ht, part_t, rmax, end;
};

struct DecodeLayout {       // moe_route / moe_expert_ffn / moe_layer, rows <= kMaxRows
  size_t logits, idx, wts, slots, order, xinv, xrec, h, part, total;
  int xrow;                 // bytes of one (format, row) block of x records
};

struct ManyRowLayout {      // moe_expert_ffn, rows > kMaxRows
  size_t xq, xs, cnt, list, chunks, n_chunks, gen, n_gen, map_gu, map_dn, hq, h32, part, total;
  int max_chunks, max_gen, max_items_gu, max_items_dn;
};

constexpr size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Shape class of a layer: 1 = hidden 5120 / inter 2304, 2 = 512 / 256, 0 = other.
inline int shape_class(const moe_dims& d) {
  if (d.hidden == 5120 && d.inter == 2304) return 1;
  if (d.hidden == 512 && d.inter == 256) return 2;
  return 0;
}

constexpr TaggedLayout tagged_layout(const moe_dims& d) {
  TaggedLayout l{};
  const size_t pairs = static_cast<size_t>(kMaxRows) * d.top_k + kMaxRows;
  size_t o = 0;
  l.err = o;      o = align256(o + 16);
  l.lgt = o;      o = align256(o + 16 * static_cast<size_t>(kMaxRows) * d.n_experts);
  l.selt = o;     o = align256(o + 8 * static_cast<size_t>(kSelRep) * kSelRepWords);
  l.ht = o;       o = align256(o + 8 * pairs * d.inter);
  l.part_t = o;   o = align256(o + 8 * pairs * d.hidden);
  // stack decode: each combine workgroup's largest |y + noise| in its row
  l.rmax = o;     o = align256(o + 8 * static_cast<size_t>(kMaxRows) * ((d.hidden + kThreads - 1) / kThreads));
  l.end = o;
  return l;
}

// The fused launch alone: the tagged area, then room for the routing outputs
// when the caller passes no idx / wts (the fixed workspace of moe_layer_noalloc).
struct FusedLayout {
  TaggedLayout t;
  size_t idx, wts, total;
};
constexpr FusedLayout fused_layout(const moe_dims& d) {
  FusedLayout l{};
  l.t = tagged_layout(d);
  size_t o = l.t.end;
  l.idx = o;      o = align256(o + 4 * static_cast<size_t>(kMaxRows) * kMaxK);
  l.wts = o;      o = align256(o + 4 * static_cast<size_t>(kMaxRows) * kMaxK);
  l.total = o;
  return l;
}

inline DecodeLayout decode_layout(const moe_dims& d, int rows) {
  DecodeLayout l{};
  const size_t pairs = static_cast<size_t>(rows) * d.top_k + rows;
  l.xrow = max_rec_row(d.hidden);
  size_t o = tagged_layout(d).end;
  l.logits = o;   o = align256(o + 8 * static_cast<size_t>(rows) * d.n_experts);
  l.idx = o;      o = align256(o + 4 * static_cast<size_t>(rows) * d.top_k);
  l.wts = o;      o = align256(o + 4 * static_cast<size_t>(rows) * d.top_k);
  l.slots = o;    o = align256(o + sizeof(SlotTable));
  l.order = o;    o = align256(o + 4 * static_cast<size_t>(rows) * d.top_k);
  l.xinv = o;     o = align256(o + 4 * static_cast<size_t>(kNumFmt) * rows);
  l.xrec = o;     o = align256(o + static_cast<size_t>(kNumFmt) * rows * l.xrow);
  l.h = o;        o = align256(o + 4 * pairs * d.inter);
  l.part = o;     o = align256(o + 4 * pairs * d.hidden);
  l.total = o;
  return l;
}

// Work items of one generic entry: channel tiles of gate/up and output tiles
// of down.  The decode tiles' largest counts over the formats, by shape class.
struct GenTiles {
  int max_gu, max_dn;
};
inline GenTiles gen_tiles(const moe_dims& d) {
  // (5120, 2304): Q8 gate/up 576 tiles of 4 channels, Q8 down 320 tiles of 16
  // outputs; (512, 256): 8 and 8.  Checked against the kernels' tile shapes
  // at compile time.
  return shape_class(d) == 1 ? GenTiles{576, 320} : GenTiles{8, 8};
}

inline ManyRowLayout many_row_layout(const moe_dims& d, int rows) {
  ManyRowLayout l{};
  const size_t R = rows, P = static_cast<size_t>(rows) * d.top_k, H = d.hidden, I = d.inter;
  const size_t PS = P + R;   // pair rows with the shared expert's
  l.max_chunks = static_cast<int>((P + kChunk - 1) / kChunk) + d.n_experts;
  l.max_gen = static_cast<int>((P + kGenRows - 1) / kGenRows) + d.n_experts +
              static_cast<int>((R + kGenRows - 1) / kGenRows);
  const GenTiles gt = gen_tiles(d);
  l.max_items_gu = l.max_gen * gt.max_gu;
  l.max_items_dn = l.max_gen * gt.max_dn;
  size_t o = tagged_layout(d).end;
  l.xq = o;       o = align256(o + R * H);
  l.xs = o;       o = align256(o + R * H / 32);
  l.cnt = o;      o = align256(o + 4 * static_cast<size_t>(d.n_experts));
  l.list = o;     o = align256(o + 4 * P);
  l.chunks = o;   o = align256(o + sizeof(Chunk) * static_cast<size_t>(l.max_chunks));
  l.n_chunks = o; o = align256(o + 4);
  l.gen = o;      o = align256(o + sizeof(GenEntry) * static_cast<size_t>(l.max_gen));
  l.n_gen = o;    o = align256(o + 16);   // entries, gate/up items, down items
  l.map_gu = o;   o = align256(o + 4 * static_cast<size_t>(l.max_items_gu));
  l.map_dn = o;   o = align256(o + 4 * static_cast<size_t>(l.max_items_dn));
  l.hq = o;       o = align256(o + 2 * P * I);
  l.h32 = o;      o = align256(o + 4 * PS * I);
  l.part = o;     o = align256(o + 4 * PS * H);
  l.total = o;
  return l;
}

}  // namespace lay
}  // namespace moe
