// Host side of the Muon C ABI: validation, the batched planner and the
// launch sequence.  See include/muon.h for the contract.
//
// Planner (RFC-0023 方案 4, muon_batch_update / muon_batch_update_size):
//  1. Every bank expands into NS units: each matrix, or each split_rows
//     block of it (RFC-0023 split_head, fan_out = head size).  Within a bank
//     the units sit at a uniform stride of rows_u*cols elements.
//  2. Units are grouped by (s, l) = (smaller, larger side) and gradient
//     dtype: a tall unit and the wide unit of the same two sides stack in
//     one pass.  The tiled products always take the tall form (rows >= cols,
//     the Gram X^T X), a unit's own choice that no batch changes, so a wide
//     unit is stored transposed in the iterate and written back transposed.
//     Wide units of at most 128 rows that the AUTO schedule may run on chip
//     keep their own form and group apart.  Every group is cut into chunks
//     of at most batch_update_size units (0 = no limit) and at most kMaxSeg
//     bank segments, transposed units after the others.
//  3. A chunk is one stacked pass: every kernel of the step runs once over
//     all of its units (and the ten NS iterations run back to back), with the
//     iterates laid out at a fixed stride in the caller's workspace.
//  4. AUTO: a pass of one 256-tile unit may ride along in a stacked pass's
//     persistent launch (pair_passes).
// The workspace is a 256-byte status header (word 0: the schedule error
// word) followed by the carve-up of the largest chunk, reused by every chunk
// (a pass with a riding pass: the two carve-ups one after the other).
#include "../../include/muon.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <tuple>
#include <vector>

#include "kernels.hpp"

using namespace muon_dev;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct Unitized {
  int desc;            // caller bank index
  int64_t n_units;     // units in the bank
  int64_t rows_u;      // unit rows
  int64_t cols;
  int32_t gdtype;
  bool trans;          // stored transposed in its chunk (a wide unit, tiled)
};

struct SegRef {
  int desc;
  int64_t unit_begin;  // first unit inside the bank
  int64_t count;
  bool trans;
};

struct Chunk {
  int64_t rows_u, cols;  // unit shape in the chunk (transposed units: caller cols x rows)
  int32_t gdtype;
  int tile;             // 128 or 256
  int64_t rows_pad, cols_pad, s_pad;
  bool tall;            // rows_u >= cols: the Gram is X^T X (every tiled chunk
                        // but one whose wide units may run on chip)
  int64_t n_units;
  int64_t n_plain;      // units 0 .. n_plain - 1 in their own form, the rest transposed
  std::vector<SegRef> segs;
  int rows_per_block, blocks_per_unit;   // momentum kernel (units in their own form)
  int tiles_t;                           // momentum kernel of transposed units: 64x64 tiles
  int partials_per_unit;                 // max of the two
  int norm_blocks_per_unit;              // 64x64 tiles of the padded iterate
  int rider = -1;  // AUTO: a one-unit pass that may run inside this pass's
                   // persistent launch (pair_passes)
  int host = -1;   // this pass may run inside pass `host`'s launch
};

// Workspace carve-up of one chunk (byte offsets).
struct Layout {
  size_t x32[2], xb[2], xt[2], a32, ab, bop, partials, inv_nu, flag, done, queue, split, total;
};

constexpr size_t kHeader = 256;  // status header at the start of the workspace
constexpr int64_t kMaxChunks = (int64_t)1 << 20;  // stacked passes per call

// Device scratch of muon_step_batched_noalloc, for callers that cannot
// allocate: a fixed array in the library's code object, one copy per GPU
// the library runs on, held until the process ends.  Host code never uses
// the array's name as an address (on the host it is only a stand-in): the
// device address comes from hipGetSymbolAddress, once per device, and is
// kept in g_scratch.
constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxQueues = 16;   // persistent schedule: at most one queue per XCC
// Passes whose momentum (fp32, 4 B per element) is larger than this take
// the non-temporal momentum kernels: the MI355X's last-level cache (the
// 256 MB Infinity Cache) cannot hold their stream.
constexpr int64_t kStreamBytes = (int64_t)256 << 20;

// Whether the AUTO schedule may run the pass on the on-chip small-unit
// kernel (bf16 products, wide units with at most 128 rows; the final choice
// also looks at the unit count and the CUs).  Only that kernel reads N in
// fp32 on the bf16 path.
bool small_possible(const Chunk& c, const muon_hyper* h) {
  if (h->schedule != MUON_SCHEDULE_AUTO || c.tall || c.rows_u > kSmall || c.rows_pad != kSmall) return false;
  // fp32 products: one-block units of at most 64 rows (their operands in
  // fp32 fill the LDS at 64 rows)
  return h->ns_precision == MUON_NS_BF16 || (c.rows_u <= 64 && c.cols_pad == kSmall);
}

// A unit that the on-chip kernels may run keeps its own (wide) form; every
// other unit takes the tall form.
bool unit_small_possible(int64_t rows_u, int64_t cols, const muon_hyper* h) {
  if (h->schedule != MUON_SCHEDULE_AUTO || rows_u >= cols || rows_u > kSmall) return false;
  return h->ns_precision == MUON_NS_BF16 || (rows_u <= 64 && cols <= kSmall);
}

// Long small units (more than eight 128-column blocks) too few to fill the
// GPU one workgroup each are split over several workgroups (at most
// kSplitMax per unit, kSplitWgMax per launch): the largest split a chunk may
// take, 1 if none.
int split_groups_max(const Chunk& c, const muon_hyper* h) {
  if (!small_possible(c, h) || h->ns_precision != MUON_NS_BF16) return 1;
  const int64_t nb = c.cols_pad / kSmall;
  if (nb <= 8 || 2 * c.n_units >= kSplitWgMax) return 1;
  return (int)std::max<int64_t>(1, std::min<int64_t>({nb, (int64_t)kSplitMax, kSplitWgMax / c.n_units}));
}

// Words of persistent-schedule completion counts per unit: three per tile
// panel on the small side.
int64_t done_words(const Chunk& c) { return 3 * (c.s_pad / c.tile); }

Layout layout_of(const Chunk& c, const muon_hyper* h) {
  const bool bf16 = h->ns_precision == MUON_NS_BF16;
  Layout L{};
  const size_t U = (size_t)c.n_units;
  const size_t xs = (size_t)(c.rows_pad * c.cols_pad);
  const size_t ss = (size_t)(c.s_pad * c.s_pad);
  size_t off = kHeader;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, kAlign); return o; };
  // fp32 iterates, fp32 path only (the bf16 path keeps the iterate in bf16,
  // and its products start from N written straight into it).
  if (!bf16) L.x32[0] = take(U * xs * 4);
  if (!bf16) L.x32[1] = take(U * xs * 4);
  if (bf16) {
    L.xb[0] = take(U * xs * 2);
    L.xb[1] = take(U * xs * 2);
  }
  // Transposed operand copies of the iterate, fp32 path only (the bf16
  // products read X itself, K-major where they need columns of X).
  if (!bf16) {
    L.xt[0] = take(U * xs * 4);
    L.xt[1] = take(U * xs * 4);
  }
  // The Gram is stored once: fp32 on the fp32 path, bf16 on the bf16 path.
  if (bf16)
    L.ab = take(U * ss * 2);
  else
    L.a32 = take(U * ss * 4);
  L.bop = take(U * ss * (bf16 ? 2 : 4));
  L.partials = take(U * (size_t)c.partials_per_unit * 8);
  L.inv_nu = take(U * 4);
  L.flag = take(U * 4);
  // persistent schedule: finished tiles per small-side tile panel, for each
  // of the three products
  L.done = take(U * done_words(c) * 4);
  L.queue = take(4 * (kMaxQueues + 1));  // persistent schedule: claim counters, leavers
  // split small units: two buffers of partial Grams per group
  const int gmax = split_groups_max(c, h);
  if (gmax > 1) L.split = take(U * 2 * (size_t)gmax * kSmall * kSmall * 4);
  L.total = off;
  return L;
}

bool finite(float x) { return std::isfinite(x); }

int validate_hyper(const muon_hyper* h) {
  if (!h) return MUON_ERR_NULL;
  if (!finite(h->lr) || !finite(h->mu) || !finite(h->weight_decay) || !finite(h->gamma))
    return MUON_ERR_HYPER;
  if (h->scale_mode != MUON_SCALE_SPECTRAL && h->scale_mode != MUON_SCALE_UNIT_RMS_NORM)
    return MUON_ERR_DTYPE;
  if (h->schedule != MUON_SCHEDULE_AUTO && h->schedule != MUON_SCHEDULE_PERSISTENT &&
      h->schedule != MUON_SCHEDULE_LAUNCHES)
    return MUON_ERR_HYPER;
  if (h->reserved != 0) return MUON_ERR_HYPER;
  if (h->nesterov_style != MUON_NESTEROV_SGD && h->nesterov_style != MUON_NESTEROV_EMA)
    return MUON_ERR_HYPER;
  if (h->nesterov_style == MUON_NESTEROV_EMA && (h->step < 1 || !(h->mu >= 0.0f && h->mu < 1.0f)))
    return MUON_ERR_HYPER;
  if (h->ns_precision != MUON_NS_FP32 && h->ns_precision != MUON_NS_BF16) return MUON_ERR_DTYPE;
  if (h->batch_update_size < 0) return MUON_ERR_HYPER;
  if (h->n_stages < 1 || h->n_stages > MUON_MAX_STAGES) return MUON_ERR_HYPER;
  int64_t total = 0;
  for (int i = 0; i < h->n_stages; ++i) {
    const muon_ns_stage& s = h->stages[i];
    if (s.steps < 0 || s.steps > 1000) return MUON_ERR_HYPER;
    if (!finite(s.a) || !finite(s.b) || !finite(s.c)) return MUON_ERR_HYPER;
    total += s.steps;
  }
  if (total < 1) return MUON_ERR_HYPER;
  return MUON_OK;
}

// Shapes: rows, cols, batch >= 1; split divides rows; kernel index limits.
int validate_descs(const muon_matrix_desc* mats, int64_t n, bool check_dtype) {
  if (n < 0) return MUON_ERR_SHAPE;
  if (n > 0 && !mats) return MUON_ERR_NULL;
  const int64_t kMaxDim = (int64_t)1 << 30;
  for (int64_t i = 0; i < n; ++i) {
    const muon_matrix_desc& d = mats[i];
    if (d.batch < 1 || d.rows < 1 || d.cols < 1 || d.split_rows < 0) return MUON_ERR_SHAPE;
    if (d.rows > kMaxDim || d.cols > kMaxDim || d.batch > kMaxDim) return MUON_ERR_SHAPE;
    if (d.split_rows > 0 && d.rows % d.split_rows != 0) return MUON_ERR_SHAPE;
    if (d.reserved != 0) return MUON_ERR_SHAPE;
    // Bytes of the largest caller bank must fit in int64 comfortably.
    const double elems = (double)d.batch * (double)d.rows * (double)d.cols;
    if (elems > 9.0e15) return MUON_ERR_SHAPE;
    if (check_dtype && d.grad_dtype != MUON_DTYPE_F32 && d.grad_dtype != MUON_DTYPE_BF16)
      return MUON_ERR_DTYPE;
  }
  return MUON_OK;
}

int pick_tile(int64_t rows_u, int64_t cols) {
  return std::min(rows_u, cols) >= 256 ? 256 : 128;
}

// AUTO: a pass of one 256-tile unit runs its three products as separate
// launches (faster than a persistent launch of its own), which leave CUs
// idle (the Gram of a 4096 x 4096 unit has 136 tiles).  It may instead
// ride along in the persistent launch of a stacked pass with the same tile
// size and operand layout (ns_persistent2), the larger such pass first,
// each stacked pass taking at most one.  Whether it does is decided per
// call on the device (run): the stacked pass must take one claim queue.
// Sides of unit shapes stay below 2^31 (validate_descs), so the trace's
// packed values hold both passes.
void pair_passes(std::vector<Chunk>* cs, const muon_hyper* h) {
  const bool bf16 = h->ns_precision == MUON_NS_BF16;
  // one operand layout per launch: bf16 wide and tall units read X
  // differently (fp32 units all read rows of X and X^T)
  auto layout = [&](const Chunk& c) { return bf16 && c.tall ? 1 : 0; };
  auto work = [](const Chunk& c) {
    return (double)c.n_units * (double)c.s_pad * (double)c.s_pad *
           (double)std::max(c.rows_pad, c.cols_pad);
  };
  // Stacked passes that may take a rider, per operand layout, largest
  // first (ties in pass order); each takes at most one, riders in pass
  // order.  (Sorting once keeps plans of many passes linear-logarithmic.)
  std::vector<int> hosts[2];
  for (size_t i = 0; i < cs->size(); ++i) {
    const Chunk& p = (*cs)[i];
    if (p.tile == 256 && p.n_units >= 2 && !small_possible(p, h)) hosts[layout(p)].push_back((int)i);
  }
  for (auto& v : hosts)
    std::stable_sort(v.begin(), v.end(),
                     [&](int x, int y) { return work((*cs)[(size_t)x]) > work((*cs)[(size_t)y]); });
  size_t next[2] = {0, 0};
  for (size_t j = 0; j < cs->size(); ++j) {
    Chunk& q = (*cs)[j];
    if (q.tile != 256 || q.n_units != 1 || small_possible(q, h) || q.segs.size() > (size_t)kMaxSegB)
      continue;
    const int k = layout(q);
    if (next[k] == hosts[k].size()) continue;
    const int best = hosts[k][next[k]++];
    (*cs)[(size_t)best].rider = (int)j;
    q.host = best;
  }
}

// Group the banks' units by shape and cut the groups into chunks.
int plan(const muon_matrix_desc* mats, int64_t n, const muon_hyper* h, bool step,
         std::vector<Chunk>* chunks) {
  std::vector<Unitized> us;
  us.reserve((size_t)n);
  for (int64_t i = 0; i < n; ++i) {
    const muon_matrix_desc& d = mats[i];
    Unitized u;
    u.desc = (int)i;
    const int64_t ru = d.split_rows > 0 ? d.split_rows : d.rows;
    u.n_units = d.batch * (d.rows / ru);
    u.gdtype = step ? d.grad_dtype : MUON_DTYPE_F32;
    // the unit's shape in its chunk: its own, or transposed to the tall form
    u.trans = ru < d.cols && !unit_small_possible(ru, d.cols, h);
    u.rows_u = u.trans ? d.cols : ru;
    u.cols = u.trans ? ru : d.cols;
    us.push_back(u);
  }
  // Group in order of first appearance, the units in their own form first
  // within each group (a chunk's transposed units follow the others).
  std::map<std::tuple<int64_t, int64_t, int32_t>, int> gid;
  std::vector<std::vector<int>> groups;
  for (int pass = 0; pass < 2; ++pass) {
    for (size_t i = 0; i < us.size(); ++i) {
      if (us[i].trans != (pass == 1)) continue;
      auto key = std::make_tuple(us[i].rows_u, us[i].cols, us[i].gdtype);
      auto it = gid.find(key);
      if (it == gid.end()) {
        gid.emplace(key, (int)groups.size());
        groups.push_back({(int)i});
      } else {
        groups[it->second].push_back((int)i);
      }
    }
  }
  const int64_t cap = h->batch_update_size > 0 ? h->batch_update_size : INT64_MAX;
  const int64_t kMaxUnitsPerChunk = (int64_t)1 << 24;  // grid-size guard
  // Every stacked pass is a host-side record and a series of launches: a
  // plan of more than kMaxChunks passes is refused before it is built (a
  // bank of 2^30 matrices under batch_update_size 1 would otherwise ask
  // for 2^30 records).
  int64_t n_chunks = 0;
  for (const auto& grp : groups) {
    int64_t units = 0;
    for (int ui : grp) {
      units += us[ui].n_units;  // each at most 9e15 (validate_descs)
      if (units > ((int64_t)1 << 60)) return MUON_ERR_SHAPE;
    }
    n_chunks += (units + std::min(cap, kMaxUnitsPerChunk) - 1) / std::min(cap, kMaxUnitsPerChunk);
    if (n_chunks > kMaxChunks) return MUON_ERR_SHAPE;
  }
  for (const auto& grp : groups) {
    const Unitized& u0 = us[grp[0]];
    Chunk proto;
    proto.rows_u = u0.rows_u;
    proto.cols = u0.cols;
    proto.gdtype = u0.gdtype;
    proto.tile = pick_tile(u0.rows_u, u0.cols);
    proto.rows_pad = round_up(u0.rows_u, proto.tile);
    proto.cols_pad = round_up(u0.cols, proto.tile);
    proto.tall = u0.rows_u >= u0.cols;
    proto.s_pad = proto.tall ? proto.cols_pad : proto.rows_pad;
    proto.n_units = 0;
    proto.n_plain = 0;
    // Momentum kernel: about 8K elements per block (measured on 32 x 1024^2
    // units: 2K per block ran at 0.65x the speed, 4K-8K fastest, 16K 6%
    // slower, 64K 25% slower); transposed units one 64x64 tile of the
    // padded caller matrix per block.
    proto.rows_per_block = (int)std::max<int64_t>(1, std::min<int64_t>(u0.rows_u, 8192 / u0.cols));
    proto.blocks_per_unit = (int)((u0.rows_u + proto.rows_per_block - 1) / proto.rows_per_block);
    proto.tiles_t = (int)((proto.rows_pad / 64) * (proto.cols_pad / 64));
    proto.partials_per_unit = proto.blocks_per_unit;
    proto.norm_blocks_per_unit = (int)((proto.rows_pad / 64) * (proto.cols_pad / 64));
    Chunk cur = proto;
    for (int ui : grp) {
      const Unitized& u = us[ui];
      int64_t begin = 0;
      while (begin < u.n_units) {
        const int64_t room = std::min(cap, kMaxUnitsPerChunk) - cur.n_units;
        if (room == 0 || (int)cur.segs.size() == kMaxSeg) {
          if ((int64_t)chunks->size() >= kMaxChunks) return MUON_ERR_SHAPE;
          chunks->push_back(cur);
          cur = proto;
          continue;
        }
        const int64_t take = std::min(room, u.n_units - begin);
        cur.segs.push_back({u.desc, begin, take, u.trans});
        cur.n_units += take;
        if (!u.trans) cur.n_plain += take;
        if (u.trans) cur.partials_per_unit = std::max(cur.partials_per_unit, cur.tiles_t);
        begin += take;
      }
    }
    if (cur.n_units > 0) chunks->push_back(cur);
  }
  // Grid-size limits of the launches, and the 2 GiB reach of the per-tile
  // buffer resources that stream K-contiguous operands (TILE rows of fp32).
  for (const Chunk& c : *chunks) {
    if ((int64_t)c.tile * std::max(c.cols_pad, c.s_pad) * 4 >= ((int64_t)1 << 31))
      return MUON_ERR_SHAPE;
    const int64_t tiles = (c.s_pad / c.tile) * (std::max(c.rows_pad, c.cols_pad) / c.tile);
    if (c.n_units * tiles > INT32_MAX / 2) return MUON_ERR_SHAPE;
    if (c.n_units * (int64_t)c.blocks_per_unit > INT32_MAX / 2) return MUON_ERR_SHAPE;
    if (c.n_units * (int64_t)c.tiles_t > INT32_MAX / 2) return MUON_ERR_SHAPE;
    if (c.n_units * (int64_t)c.norm_blocks_per_unit > INT32_MAX / 2) return MUON_ERR_SHAPE;
    // a K-major bf16 operand tile spans every row of the iterate
    if (c.rows_pad * c.cols_pad * 2 >= ((int64_t)1 << 31)) return MUON_ERR_SHAPE;
  }
  if (h->schedule == MUON_SCHEDULE_AUTO) pair_passes(chunks, h);
  return MUON_OK;
}

// riding: room for riding passes (every call but the scratch entry's,
// whose passes never ride along).
size_t workspace_of(const std::vector<Chunk>& chunks, const muon_hyper* h, bool riding = true) {
  size_t need = kHeader;
  for (const Chunk& c : chunks) {
    size_t t = layout_of(c, h).total;
    // a riding pass's buffers follow the stacked pass's
    if (riding && c.rider >= 0) t += layout_of(chunks[(size_t)c.rider], h).total - kHeader;
    need = std::max(need, t);
  }
  return need;
}

// M <- ma*M + mb*G and N = la*M + lb*G (RFC-0023 方案 1).  SGD style: mu, 1,
// mu, 1.  EMA style: mu, 1 - mu, mu/(1 - mu^(t+1)), (1 - mu)/(1 - mu^t), the
// bias corrections evaluated in double.
void momentum_coefficients(const muon_hyper* h, float* ma, float* mb, float* la, float* lb) {
  const double mu = h->mu;
  if (h->nesterov_style == MUON_NESTEROV_EMA) {
    const double t = (double)h->step;
    *ma = (float)mu;
    *mb = (float)(1.0 - mu);
    *la = (float)(mu / (1.0 - std::pow(mu, t + 1.0)));
    *lb = (float)((1.0 - mu) / (1.0 - std::pow(mu, t)));
  } else {
    *ma = h->mu;
    *mb = 1.0f;
    *la = h->mu;
    *lb = 1.0f;
  }
}

// Update scale of a unit of fan_out x fan_in ([V4-notes]-style spectral, or
// the Megatron PR's unit_rms_norm).
double unit_scale(int64_t fan_out, int64_t fan_in, const muon_hyper* h) {
  const double fo = (double)fan_out, fi = (double)fan_in;
  if (h->scale_mode == MUON_SCALE_SPECTRAL) return std::sqrt(std::max(fo, fi)) * (double)h->gamma;
  return std::sqrt(fo / fi);
}

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

struct Range {
  uintptr_t lo, hi;
  int owner;
};

// Overlap between any two written buffers, or between a written buffer and
// an input of another bank.
int check_alias(const std::vector<Range>& written, const std::vector<Range>& read) {
  std::vector<Range> w = written;
  std::sort(w.begin(), w.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < w.size(); ++i)
    if (w[i].lo < w[i - 1].hi) return MUON_ERR_ALIAS;
  for (const Range& r : read)
    for (const Range& x : w)
      if (r.lo < x.hi && x.lo < r.hi && !(r.owner == x.owner && r.lo == x.lo && r.hi == x.hi))
        return MUON_ERR_ALIAS;
  return MUON_OK;
}

struct Tracer {
  muon_trace* t;
  hipStream_t s;
  void before(int kind) {
    if (t && t->kind == kind && t->count < t->capacity)
      (void)hipEventRecord(t->events[2 * t->count], s);
  }
  // info: what the launch covered (muon.h, muon_trace)
  void after(int kind, int64_t i0 = 0, int64_t i1 = 0, int64_t i2 = 0, int64_t i3 = 0) {
    if (t && t->kind == kind) {
      if (t->count < t->capacity) {
        (void)hipEventRecord(t->events[2 * t->count + 1], s);
        if (t->info) {
          int64_t* q = t->info + 4 * (int64_t)t->count;
          q[0] = i0;
          q[1] = i1;
          q[2] = i2;
          q[3] = i3;
        }
      }
      t->count++;
    }
  }
  // an NS launch over a chunk: smaller and larger unit side, units, tile;
  // a launch that also runs a riding pass carries that pass's three values
  // in the upper 32 bits of each (muon.h, muon_trace)
  void after_ns(int kind, const Chunk& c, const Chunk* r = nullptr) {
    auto pack = [](int64_t lo, int64_t hi) { return lo | (hi << 32); };
    after(kind, pack(std::min(c.rows_u, c.cols), r ? std::min(r->rows_u, r->cols) : 0),
          pack(std::max(c.rows_u, c.cols), r ? std::max(r->rows_u, r->cols) : 0),
          pack(c.n_units, r ? r->n_units : 0), c.tile);
  }
};

// Per-device facts the persistent launch needs: resident workgroups of each
// kernel variant and the wall-clock rate.
struct DeviceInfo {
  bool ready = false;
  int cus = 0;
  int wall_khz = 0;
  int xccs = 1;
  int resident[2][2] = {{0, 0}, {0, 0}};  // [bf16][tile 256]
};

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
DeviceInfo g_dev[kMaxDevices];

template <typename T, int TILE>
int resident_of(int cus) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ns_persistent<T, TILE, sizeof(T) == 2 ? 1 : 0>,
                                                   gemm_threads<TILE>(), 0) !=
          hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  return per_cu * cus;
}

int device_info(DeviceInfo* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MUON_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.ready) {
    if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&d.wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
        d.cus < 1 || d.wall_khz < 1)
      return MUON_ERR_HIP;
    if (hipDeviceGetAttribute(&d.xccs, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess ||
        d.xccs < 1)
      d.xccs = 1;
    d.xccs = std::min(d.xccs, kMaxQueues);
    d.resident[0][0] = resident_of<float, 128>(d.cus);
    d.resident[0][1] = resident_of<float, 256>(d.cus);
    d.resident[1][0] = resident_of<__bf16, 128>(d.cus);
    d.resident[1][1] = resident_of<__bf16, 256>(d.cus);
    d.ready = true;
  }
  *out = d;
  return MUON_OK;
}

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's copy of `scratch` (its address looked up on the
// first call on the device).
int scratch_workspace(void** ws, size_t* bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MUON_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MUON_ERR_HIP;
    g_scratch[dev] = p;
  }
  *ws = g_scratch[dev];
  *bytes = kScratchBytes;
  return MUON_OK;
}

constexpr double kWaitLimitSeconds = 5.0;  // bound of one dependency wait

// Bound of one dependency wait in wall-clock ticks.  Test hook:
// MUON_WAIT_LIMIT_US replaces the 5 s bound (0 = give up as soon as a wait
// does not succeed at once), so that tests can drive the schedule's stop
// path from the host while every kernel still exits normally.
uint64_t wait_limit_ticks(int wall_khz) {
  double seconds = kWaitLimitSeconds;
  if (const char* us = std::getenv("MUON_WAIT_LIMIT_US")) {
    char* end = nullptr;
    const double v = std::strtod(us, &end);
    if (end != us && v >= 0.0 && v < 1e9) seconds = v * 1e-6;
  }
  return (uint64_t)(seconds * 1e3 * (double)wall_khz);
}

template <int PHASE, typename T, int KM>
void launch_gemm(int tile, const GemmArgs& g, const ChunkArgs& ca, hipStream_t s) {
  const int per_unit = g.sym ? g.tiles_m * (g.tiles_m + 1) / 2 : g.tiles_m * g.tiles_n;
  const int grid = g.n_units * per_unit;
  if (tile == 256)
    hipLaunchKernelGGL((ns_gemm<PHASE, T, 256, KM>), dim3(grid), dim3(gemm_threads<256>()), 0, s, g, ca);
  else
    hipLaunchKernelGGL((ns_gemm<PHASE, T, 128, KM>), dim3(grid), dim3(gemm_threads<128>()), 0, s, g, ca);
}

// km: bit 0 = the A operand is K-major, bit 1 = the B operand is (bf16 only).
template <int PHASE>
void launch_phase(bool bf16, int tile, int km, const GemmArgs& g, const ChunkArgs& ca, hipStream_t s) {
  if (!bf16)
    launch_gemm<PHASE, float, 0>(tile, g, ca, s);
  else if (km == 3)
    launch_gemm<PHASE, __bf16, 3>(tile, g, ca, s);
  else if (km == 2)
    launch_gemm<PHASE, __bf16, 2>(tile, g, ca, s);
  else
    launch_gemm<PHASE, __bf16, 0>(tile, g, ca, s);
}

// The chunk's kernel arguments: its shape, the momentum coefficients and
// the caller matrices of its units.
void fill_chunk_args(ChunkArgs* ca, const Chunk& c, const muon_hyper* h, bool step,
                     float* const* outs, const void* const* ins, float* const* moms,
                     const muon_matrix_desc* mats) {
  std::memset(ca, 0, sizeof(*ca));
  ca->n_seg = (int32_t)c.segs.size();
  ca->n_units = (int32_t)c.n_units;
  ca->rows = (int32_t)c.rows_u;
  ca->cols = (int32_t)c.cols;
  ca->rows_pad = (int32_t)c.rows_pad;
  ca->cols_pad = (int32_t)c.cols_pad;
  ca->unit_elems = c.rows_u * c.cols;
  ca->x_stride = c.rows_pad * c.cols_pad;
  momentum_coefficients(h, &ca->ma, &ca->mb, &ca->la, &ca->lb);
  ca->decay = (float)(1.0 - (double)h->lr * (double)h->weight_decay);
  ca->lr_scale = (float)((double)h->lr * unit_scale(c.rows_u, c.cols, h));
  const float lr_scale_t = (float)((double)h->lr * unit_scale(c.cols, c.rows_u, h));
  int32_t first = 0;
  for (size_t i = 0; i < c.segs.size(); ++i) {
    const SegRef& r = c.segs[i];
    const int64_t off = r.unit_begin * c.rows_u * c.cols;  // elements
    ca->seg[i].w = outs[r.desc] + off;
    const size_t gsz = (step && mats[r.desc].grad_dtype == MUON_DTYPE_BF16) ? 2 : 4;
    ca->seg[i].g = static_cast<const unsigned char*>(ins[r.desc]) + off * (int64_t)gsz;
    ca->seg[i].m = step ? moms[r.desc] + off : nullptr;
    ca->seg[i].first = first;
    ca->seg[i].count = (int32_t)r.count;
    ca->seg[i].trans = r.trans ? 1 : 0;
    // a transposed unit's fan_out is the chunk's cols
    ca->seg[i].lr_scale = r.trans ? lr_scale_t : ca->lr_scale;
    first += (int32_t)r.count;
  }
}

// A chunk's buffers in the workspace.  `base` is where its layout's offsets
// count from: the workspace itself, or, for a pass riding along in another
// pass's launch, the end of that pass's buffers (less the header).
struct ChunkBufs {
  Layout L;
  float* x32[2];
  uint16_t* xb[2];
  void* xt[2];
  float* a32;
  uint16_t* ab;
  void* bop;
  double* partials;
  float* inv_nu;
  int32_t* flag;
  uint32_t* done;
  uint32_t* queue;
  void* split;
};

ChunkBufs chunk_bufs(const Chunk& c, const muon_hyper* h, unsigned char* base) {
  const bool bf16 = h->ns_precision == MUON_NS_BF16;
  ChunkBufs B;
  B.L = layout_of(c, h);
  const Layout& L = B.L;
  B.x32[0] = L.x32[0] ? reinterpret_cast<float*>(base + L.x32[0]) : nullptr;
  B.x32[1] = bf16 ? nullptr : reinterpret_cast<float*>(base + L.x32[1]);
  B.xb[0] = bf16 ? reinterpret_cast<uint16_t*>(base + L.xb[0]) : nullptr;
  B.xb[1] = bf16 ? reinterpret_cast<uint16_t*>(base + L.xb[1]) : nullptr;
  B.xt[0] = bf16 ? nullptr : base + L.xt[0];
  B.xt[1] = bf16 ? nullptr : base + L.xt[1];
  B.a32 = bf16 ? nullptr : reinterpret_cast<float*>(base + L.a32);
  B.ab = bf16 ? reinterpret_cast<uint16_t*>(base + L.ab) : nullptr;
  B.bop = base + L.bop;
  B.partials = reinterpret_cast<double*>(base + L.partials);
  B.inv_nu = reinterpret_cast<float*>(base + L.inv_nu);
  B.flag = reinterpret_cast<int32_t*>(base + L.flag);
  B.done = reinterpret_cast<uint32_t*>(base + L.done);
  B.queue = reinterpret_cast<uint32_t*>(base + L.queue);
  B.split = L.split ? base + L.split : nullptr;
  return B;
}

// Steps 1 and 2 of a tiled or streamed pass: momentum (or the NS-input
// copy) with the partial sums of squares, the norm finish, and, off the
// folded path, X0 = N / ||N||_F.  `err`: the call's status word when this
// is the first pass of the call (the norm finish clears it), else nullptr.
void launch_prologue(const Chunk& c, const ChunkArgs& ca, const ChunkBufs& B, const muon_hyper* h,
                     bool step, uint32_t* err, hipStream_t s, Tracer& tr) {
  const bool bf16 = h->ns_precision == MUON_NS_BF16;
  // The bf16 paths fold 1/nu into the first iteration: momentum writes N
  // straight into the bf16 iterate (padding zeroed) and no normalisation
  // pass runs.
  uint16_t* const nb = bf16 ? B.xb[0] : nullptr;
  const int gk = !step ? 2 : (c.gdtype == MUON_DTYPE_BF16 ? 0 : 1);
  // Units in their own form (0 .. n_plain - 1), then transposed ones; each
  // launch's algorithmic bytes: G (or the NS input) read, M read and
  // written (step), N written into the bf16 iterate (2 B) or in fp32 (4 B).
  const int64_t pp = c.partials_per_unit;
  auto mom_info = [&](int64_t units) {
    const int64_t elems = units * c.rows_u * c.cols;
    const int64_t gsz = (step && c.gdtype == MUON_DTYPE_BF16) ? 2 : 4;
    const int64_t per = gsz + (step ? 8 : 0) + (nb ? 2 : 4);
    tr.after(MUON_KERNEL_MOMENTUM, elems, elems * per, units, 0);
  };
  float* const x0 = B.x32[0];
  double* const partials = B.partials;
  // Non-temporal gradient and momentum accesses for passes whose momentum
  // (or NS input) outgrows the last-level cache (kernels.hpp, ld_f4).
  const bool nt = c.n_units * c.rows_u * c.cols * 4 > kStreamBytes;
  if (c.n_plain > 0) {
    tr.before(MUON_KERNEL_MOMENTUM);
    const dim3 grid((unsigned)(c.n_plain * c.blocks_per_unit));
    const int bpu = c.blocks_per_unit, rpb = c.rows_per_block;
#define MUON_MOMENTUM(GK, NT) \
  hipLaunchKernelGGL((k_momentum<GK, NT>), grid, dim3(kThreads), 0, s, ca, x0, nb, partials, rpb, bpu, 0, (int)pp)
    if (gk == 2)
      { if (nt) MUON_MOMENTUM(2, true); else MUON_MOMENTUM(2, false); }
    else if (gk == 0)
      { if (nt) MUON_MOMENTUM(0, true); else MUON_MOMENTUM(0, false); }
    else
      { if (nt) MUON_MOMENTUM(1, true); else MUON_MOMENTUM(1, false); }
#undef MUON_MOMENTUM
    mom_info(c.n_plain);
  }
  if (c.n_units > c.n_plain) {
    tr.before(MUON_KERNEL_MOMENTUM);
    const dim3 grid((unsigned)((c.n_units - c.n_plain) * c.tiles_t));
    const int u0 = (int)c.n_plain;
#define MUON_MOMENTUM_T(GK, NT) \
  hipLaunchKernelGGL((k_momentum_t<GK, NT>), grid, dim3(kThreads), 0, s, ca, x0, nb, partials, u0, (int)pp)
    if (gk == 2)
      { if (nt) MUON_MOMENTUM_T(2, true); else MUON_MOMENTUM_T(2, false); }
    else if (gk == 0)
      { if (nt) MUON_MOMENTUM_T(0, true); else MUON_MOMENTUM_T(0, false); }
    else
      { if (nt) MUON_MOMENTUM_T(1, true); else MUON_MOMENTUM_T(1, false); }
#undef MUON_MOMENTUM_T
    mom_info(c.n_units - c.n_plain);
  }
  // norms (and, off the folded path, X0 = N / ||N||_F)
  tr.before(MUON_KERNEL_NORMALIZE);
  hipLaunchKernelGGL(k_norm_finish, dim3((unsigned)c.n_units), dim3(kThreads), 0, s, partials,
                     (int)pp, B.inv_nu, B.flag, B.done, (int)done_words(c), B.queue,
                     kMaxQueues + 1, err, nb, (int64_t)(c.rows_pad * c.cols_pad));
  if (!bf16)
    hipLaunchKernelGGL(k_normalize, dim3((unsigned)(c.n_units * c.norm_blocks_per_unit)),
                       dim3(kThreads), 0, s, ca, x0, static_cast<float*>(B.xt[0]), B.inv_nu,
                       (int)(c.cols_pad / 64), c.norm_blocks_per_unit);
  tr.after(MUON_KERNEL_NORMALIZE, c.n_units);
}

// Symmetric tiles per unit (upper triangle) and apply tiles per unit.
int sym_tiles(const Chunk& c) {
  const int64_t t = c.s_pad / c.tile;
  return (int)(t * (t + 1) / 2);
}
int apply_tiles(const Chunk& c) { return (int)((c.rows_pad / c.tile) * (c.cols_pad / c.tile)); }

// The persistent schedule's description of one pass: its three products
// and where its tiles are counted.
void fill_pass(NsPass* P, const Chunk& c, const ChunkBufs& B, const muon_hyper* h) {
  const bool bf16 = h->ns_precision == MUON_NS_BF16;
  std::memset(P, 0, sizeof(*P));
  const int U = (int)c.n_units;
  const int T = c.tile;
  const int64_t xs = c.rows_pad * c.cols_pad;
  const int64_t ss = c.s_pad * c.s_pad;
  const int64_t sp = c.s_pad;
  // Operand copies of the iterate: X as is (bf16, or the fp32 iterate
  // itself) and, on the fp32 path only, X^T (cols_pad x rows_pad); the bf16
  // products read X K-major instead.
  const void* xop[2] = {bf16 ? (const void*)B.xb[0] : (const void*)B.x32[0],
                        bf16 ? (const void*)B.xb[1] : (const void*)B.x32[1]};
  const void* aop = bf16 ? (const void*)B.ab : (const void*)B.a32;
  // First iteration's scale on the folded path (inv_nu as k_norm_finish
  // left it): Gram by its square, apply by itself.
  const float* const fold_scale = bf16 ? B.inv_nu : nullptr;
  // Gram: A = X X^T (wide, rows of X) or X^T X (tall, rows of X^T).
  // bf16: a tall unit's X^T X reads X K-major; fp32: rows of X^T.
  GemmArgs& gg = P->gram;
  gg.n_units = U;
  gg.flag = B.flag;
  gg.fold = fold_scale;  // the kernel keeps it for the first iteration only
  gg.a_ustride = gg.b_ustride = xs;
  gg.lda = gg.ldb = (int32_t)(c.tall && !bf16 ? c.rows_pad : c.cols_pad);
  gg.M = gg.N = (int32_t)sp;
  gg.K = (int32_t)(c.tall ? c.rows_pad : c.cols_pad);
  gg.tiles_m = gg.tiles_n = (int32_t)(sp / T);
  gg.sym = 1;
  gg.out32 = B.a32;
  gg.out16 = B.ab;
  gg.out_ustride = ss;
  gg.ldo = (int32_t)sp;
  for (int k = 0; k < 2; ++k) P->gram_op[k] = c.tall && !bf16 ? (const void*)B.xt[k] : xop[k];
  // Polynomial: B' = a*I + b*A + c*A*A (the apply's a*X term on its
  // diagonal; a comes per iteration).
  GemmArgs& gp = P->poly;
  gp.n_units = U;
  gp.flag = B.flag;
  gp.a = gp.b = aop;
  gp.a_ustride = gp.b_ustride = ss;
  gp.lda = gp.ldb = (int32_t)sp;
  gp.M = gp.N = gp.K = (int32_t)sp;
  gp.tiles_m = gp.tiles_n = (int32_t)(sp / T);
  gp.sym = 1;
  gp.out32 = bf16 ? nullptr : static_cast<float*>(B.bop);
  gp.out16 = bf16 ? B.bop : nullptr;
  gp.out_ustride = ss;
  gp.ldo = (int32_t)sp;
  gp.aux = B.a32;
  gp.aux16 = B.ab;
  gp.aux_ustride = ss;
  gp.ldaux = (int32_t)sp;
  // Apply: X' = B'*X (wide) or X*B' (tall).
  GemmArgs& ga = P->apply;
  ga.n_units = U;
  ga.flag = B.flag;
  ga.fold = fold_scale;
  ga.M = (int32_t)c.rows_pad;
  ga.N = (int32_t)c.cols_pad;
  ga.K = (int32_t)sp;
  ga.tiles_m = (int32_t)(c.rows_pad / T);
  ga.tiles_n = (int32_t)(c.cols_pad / T);
  if (!c.tall) {
    ga.a_ustride = ss;
    ga.lda = (int32_t)sp;
    ga.b_ustride = xs;
    ga.ldb = (int32_t)(bf16 ? c.cols_pad : c.rows_pad);  // X K-major, or rows of X^T
  } else {
    ga.a_ustride = xs;
    ga.lda = (int32_t)c.cols_pad;
    ga.b_ustride = ss;
    ga.ldb = (int32_t)sp;
  }
  ga.out_ustride = xs;
  ga.ldo = (int32_t)c.cols_pad;
  ga.ldt = (int32_t)c.rows_pad;
  for (int k = 0; k < 2; ++k) {
    const int nx = k ^ 1;
    P->app_a[k] = c.tall ? xop[k] : (const void*)B.bop;
    P->app_b[k] = c.tall ? (const void*)B.bop : (bf16 ? xop[k] : (const void*)B.xt[k]);
    P->app_out32[k] = bf16 ? nullptr : B.x32[nx];
    P->app_out16[k] = bf16 ? (void*)B.xb[nx] : nullptr;
    P->app_outt[k] = B.xt[nx];  // nullptr on the bf16 path
  }
  P->done = B.done;
  P->n_units = U;
  P->tg = sym_tiles(c);
  P->ta = apply_tiles(c);
  P->apply_s_m = c.tall ? 0 : 1;
}

// Claim queues of a persistent launch over `units` units: one per XCC when
// the units spread over the XCCs with at most an eighth of the slots idle,
// one otherwise.
int queues_for(int64_t units, int xccs) {
  const int64_t slots = (units + xccs - 1) / xccs * (int64_t)xccs;
  return (xccs > 1 && units >= xccs && 8 * (slots - units) <= slots) ? xccs : 1;
}

// Work items of a pass's persistent schedule.
int64_t persistent_items(const Chunk& c, int n_iter) {
  return (int64_t)n_iter * c.n_units * (2 * (int64_t)sym_tiles(c) + apply_tiles(c));
}

// Runs one chunk: momentum (or NS-input copy), norms, normalisation (folded
// into the first iteration on the bf16 paths) and the NS iterations with the
// fused final epilogue; units of one 128 x 128 block take all of it in one
// launch.  `rider`: a one-unit pass whose products run inside this chunk's
// persistent launch (pair_passes; its buffers follow this chunk's in the
// workspace).
int run_chunk(const Chunk& c, const muon_hyper* h, bool step, float* const* outs,
              const void* const* ins, float* const* moms, const muon_matrix_desc* mats,
              unsigned char* ws, hipStream_t s, Tracer& tr, bool first_chunk,
              bool allow_waits, const Chunk* rider = nullptr) {
  const bool bf16 = h->ns_precision == MUON_NS_BF16;
  ChunkArgs ca;
  fill_chunk_args(&ca, c, h, step, outs, ins, moms, mats);
  const ChunkBufs B = chunk_bufs(c, h, ws);
  const Layout& L = B.L;
  uint16_t* const* xb = B.xb;

  const int U = (int)c.n_units;
  // Small wide units (AUTO schedule; at most 128 rows with bf16 products,
  // at most 64 rows and 128 columns with fp32 ones): the whole NS in one
  // workgroup per unit.  A unit's workgroup walks its column blocks in
  // sequence, so the path is taken for short units (up to eight 128-column
  // blocks) or when the units number at least half the CUs; a few long
  // units go to the tiled products, which spread each unit over many CUs.
  bool small = small_possible(c, h);
  int groups = 1;            // workgroups per unit on the on-chip path
  uint64_t wait_ticks = 0;
  if (small && c.cols_pad / kSmall > 8) {
    DeviceInfo di;
    const int dst = device_info(&di);
    if (dst != MUON_OK) return dst;
    if (2 * U < di.cus) {
      // Too few to fill the GPU one workgroup each: split each unit over
      // several (their groups wait on each other, so only where waits are
      // allowed and every workgroup of the launch gets a CU of its own),
      // else the tiled products.
      const int gmax = split_groups_max(c, h);
      groups = std::min(gmax, di.cus / U);
      small = allow_waits && groups > 1;
      wait_ticks = wait_limit_ticks(di.wall_khz);
    }
  }
  const int gk = !step ? 2 : (c.gdtype == MUON_DTYPE_BF16 ? 0 : 1);
  auto small_args = [&]() {
    NsSmallArgs p;
    std::memset(&p, 0, sizeof(p));
    p.xb[0] = xb[0];
    p.xb[1] = xb[1];
    p.x_stride = c.rows_pad * c.cols_pad;
    p.ldx = (int32_t)c.cols_pad;
    p.n_stages = h->n_stages;
    int begin = 0;
    for (int i = 0; i < h->n_stages; ++i) {
      p.stage_begin[i] = begin;
      begin += h->stages[i].steps;
      p.sa[i] = h->stages[i].a;
      p.sb[i] = h->stages[i].b;
      p.sc[i] = h->stages[i].c;
    }
    p.n_iter = begin;
    p.final_mode = step ? FINAL_STEP : FINAL_NSOUT;
    p.inv_nu = B.inv_nu;
    p.flag = B.flag;
    p.groups = 1;
    return p;
  };
  // Units of one 128 x 128 block: the whole step in one launch, over the
  // unit's extent in 32-row and 32-column blocks.
  if (small && c.cols_pad == kSmall) {
    const NsSmallArgs p = small_args();
    uint32_t* err = first_chunk ? reinterpret_cast<uint32_t*>(ws) : nullptr;
    const int bs = (int)((c.rows_u + 31) / 32), bl = (int)((c.cols + 31) / 32);
    tr.before(MUON_KERNEL_NS_SMALL);
    const dim3 grid(U), block(kThreads);
#define MUON_SMALL_STEP(T, BS, BL) \
  case BS * 8 + BL:                \
    hipLaunchKernelGGL((k_ns_small_step<T, BS, BL>), grid, block, 0, s, p, ca, gk, err); \
    break;
    if (bf16) {
      switch (bs * 8 + bl) {
        MUON_SMALL_STEP(__bf16, 1, 1) MUON_SMALL_STEP(__bf16, 1, 2) MUON_SMALL_STEP(__bf16, 1, 3)
        MUON_SMALL_STEP(__bf16, 1, 4) MUON_SMALL_STEP(__bf16, 2, 2) MUON_SMALL_STEP(__bf16, 2, 3)
        MUON_SMALL_STEP(__bf16, 2, 4) MUON_SMALL_STEP(__bf16, 3, 3) MUON_SMALL_STEP(__bf16, 3, 4)
        MUON_SMALL_STEP(__bf16, 4, 4)
        default:
          return MUON_ERR_SHAPE;  // not reached: rows <= cols <= 128
      }
    } else {
      switch (bs * 8 + bl) {
        MUON_SMALL_STEP(float, 1, 1) MUON_SMALL_STEP(float, 1, 2) MUON_SMALL_STEP(float, 1, 3)
        MUON_SMALL_STEP(float, 1, 4) MUON_SMALL_STEP(float, 2, 2) MUON_SMALL_STEP(float, 2, 3)
        MUON_SMALL_STEP(float, 2, 4)
        default:
          return MUON_ERR_SHAPE;  // not reached: rows <= 64, rows <= cols <= 128
      }
    }
#undef MUON_SMALL_STEP
    tr.after_ns(MUON_KERNEL_NS_SMALL, c);
    return hipGetLastError() == hipSuccess ? MUON_OK : MUON_ERR_HIP;
  }
  // 1-2. momentum, norms (and X0 on the fp32 path); the riding pass's too.
  uint32_t* const err = reinterpret_cast<uint32_t*>(ws);
  launch_prologue(c, ca, B, h, step, first_chunk ? err : nullptr, s, tr);
  ChunkArgs ca_r;
  ChunkBufs B_r{};
  if (rider) {
    fill_chunk_args(&ca_r, *rider, h, step, outs, ins, moms, mats);
    B_r = chunk_bufs(*rider, h, ws + (L.total - kHeader));
    launch_prologue(*rider, ca_r, B_r, h, step, nullptr, s, tr);
  }
  if (small) {
    NsSmallArgs p = small_args();
    if (groups > 1) {
      p.groups = groups;
      p.cnt = B.done;
      p.cnt_stride = (int32_t)done_words(c);
      p.part = static_cast<float*>(B.split);
      p.err = err;
      p.timeout_ticks = wait_ticks;
    }
    tr.before(MUON_KERNEL_NS_SMALL);
    hipLaunchKernelGGL(k_ns_small, dim3(U * groups), dim3(kThreads), 0, s, p, ca);
    tr.after_ns(MUON_KERNEL_NS_SMALL, c);
    return hipGetLastError() == hipSuccess ? MUON_OK : MUON_ERR_HIP;
  }

  // 3. Newton-Schulz iterations.
  const int T = c.tile;
  const int64_t xs = c.rows_pad * c.cols_pad;
  const int64_t ss = c.s_pad * c.s_pad;
  const int64_t sp = c.s_pad;
  const void* xop[2] = {bf16 ? (const void*)xb[0] : (const void*)B.x32[0],
                        bf16 ? (const void*)xb[1] : (const void*)B.x32[1]};
  const void* aop = bf16 ? (const void*)B.ab : (const void*)B.a32;
  const float* const fold_scale = bf16 ? B.inv_nu : nullptr;
  int total = 0;
  for (int i = 0; i < h->n_stages; ++i) total += h->stages[i].steps;
  const int64_t n_items = persistent_items(c, total) + (rider ? persistent_items(*rider, total) : 0);
  // AUTO: persistent for 256-tile passes of two units or more.  128-tile
  // passes (short K) run faster as separate launches than as claimed
  // tiles, and so does a pass of one unit on its own, whose phases cannot
  // overlap another unit's and whose single claim queue publishes every
  // tile through memory (one 4096 x 4096 unit: 3.1 ms as launches, 3.6-3.9
  // ms persistent; two units: 6.4 ms against 5.4 ms).  Such a pass runs
  // inside a stacked pass's launch instead where one fits (`rider`).
  const bool persistent = allow_waits && (h->schedule == MUON_SCHEDULE_PERSISTENT ||
                                          (h->schedule == MUON_SCHEDULE_AUTO && T == 256 && U >= 2));
  if (rider && !(persistent && n_items < INT32_MAX / 2)) return MUON_ERR_SCHEDULE;  // not reached
  if (persistent && n_items < INT32_MAX / 2) {
    DeviceInfo di;
    const int dst = device_info(&di);
    if (dst != MUON_OK) return dst;
    NsSched p;
    std::memset(&p, 0, sizeof(p));
    fill_pass(&p.a, c, B, h);
    p.final_mode = step ? FINAL_STEP : FINAL_NSOUT;
    p.n_iter = total;
    p.n_stages = h->n_stages;
    int begin = 0;
    for (int i = 0; i < h->n_stages; ++i) {
      p.stage_begin[i] = begin;
      begin += h->stages[i].steps;
      p.sa[i] = h->stages[i].a;
      p.sb[i] = h->stages[i].b;
      p.sc[i] = h->stages[i].c;
    }
    // A stage with zero steps begins where the next one does; the kernel
    // takes the last stage whose beginning it has reached.
    p.n_queues = rider ? 1 : queues_for(U, di.xccs);
    p.queue = B.queue;
    p.err = err;
    p.timeout_ticks = wait_limit_ticks(di.wall_khz);
    int grid = (int)std::min<int64_t>(n_items, di.resident[bf16 ? 1 : 0][T == 256 ? 1 : 0]);
    // Test hook: MUON_PERSISTENT_WORKGROUPS caps the grid, so that tests can
    // run the schedule with XCCs that receive no workgroup.
    if (const char* cap = std::getenv("MUON_PERSISTENT_WORKGROUPS")) {
      const int c = std::atoi(cap);
      if (c > 0) grid = std::min(grid, c);
    }
    tr.before(MUON_KERNEL_NS);
    if (rider) {
      NsPassB pb;
      std::memset(&pb, 0, sizeof(pb));
      fill_pass(&pb.b, *rider, B_r, h);
      pb.rows = ca_r.rows;
      pb.cols = ca_r.cols;
      pb.unit_elems = ca_r.unit_elems;
      pb.decay = ca_r.decay;
      pb.n_seg = ca_r.n_seg;
      for (int i = 0; i < ca_r.n_seg; ++i) pb.seg[i] = ca_r.seg[i];  // n_seg <= kMaxSegB
      const dim3 g3(grid), b3(gemm_threads<256>());
      if (bf16 && !c.tall)
        hipLaunchKernelGGL((ns_persistent2<__bf16, 256, 1>), g3, b3, 0, s, p, ca, pb);
      else if (bf16)
        hipLaunchKernelGGL((ns_persistent2<__bf16, 256, 2>), g3, b3, 0, s, p, ca, pb);
      else
        hipLaunchKernelGGL((ns_persistent2<float, 256, 0>), g3, b3, 0, s, p, ca, pb);
      tr.after_ns(MUON_KERNEL_NS, c, rider);
    } else {
      if (bf16 && !c.tall) {
        if (T == 256)
          hipLaunchKernelGGL((ns_persistent<__bf16, 256, 1>), dim3(grid), dim3(gemm_threads<256>()), 0, s, p, ca);
        else
          hipLaunchKernelGGL((ns_persistent<__bf16, 128, 1>), dim3(grid), dim3(gemm_threads<128>()), 0, s, p, ca);
      } else if (bf16) {
        if (T == 256)
          hipLaunchKernelGGL((ns_persistent<__bf16, 256, 2>), dim3(grid), dim3(gemm_threads<256>()), 0, s, p, ca);
        else
          hipLaunchKernelGGL((ns_persistent<__bf16, 128, 2>), dim3(grid), dim3(gemm_threads<128>()), 0, s, p, ca);
      } else {
        if (T == 256)
          hipLaunchKernelGGL((ns_persistent<float, 256, 0>), dim3(grid), dim3(gemm_threads<256>()), 0, s, p, ca);
        else
          hipLaunchKernelGGL((ns_persistent<float, 128, 0>), dim3(grid), dim3(gemm_threads<128>()), 0, s, p, ca);
      }
      tr.after_ns(MUON_KERNEL_NS, c);
    }
    return hipGetLastError() == hipSuccess ? MUON_OK : MUON_ERR_HIP;
  }
  float* const* x32 = B.x32;
  void* const* xt = B.xt;
  float* const a32 = B.a32;
  uint16_t* const ab = B.ab;
  void* const bop = B.bop;
  int32_t* const flag = B.flag;
  int it = 0;
  for (int st = 0; st < h->n_stages; ++st) {
    const muon_ns_stage& sg = h->stages[st];
    for (int k = 0; k < sg.steps; ++k, ++it) {
      const int cur = it & 1, nxt = cur ^ 1;
      const bool last = (it == total - 1);
      // Gram: A = X X^T (wide) or X^T X (tall), s_pad x s_pad.
      GemmArgs g;
      std::memset(&g, 0, sizeof(g));
      g.n_units = U;
      g.flag = flag;
      // wide: rows of X (K = cols); tall: X K-major (bf16) or rows of X^T
      // (fp32), K = rows
      g.a = c.tall && !bf16 ? (const void*)xt[cur] : xop[cur];
      g.b = g.a;
      g.a_ustride = g.b_ustride = xs;
      g.lda = g.ldb = (int32_t)(c.tall && !bf16 ? c.rows_pad : c.cols_pad);
      g.M = g.N = (int32_t)sp;
      g.K = (int32_t)(c.tall ? c.rows_pad : c.cols_pad);
      g.tiles_m = g.tiles_n = (int32_t)(sp / T);
      g.sym = 1;       // A is symmetric: upper-triangle tiles, mirrored
      g.fold = it == 0 ? fold_scale : nullptr;
      g.out32 = a32;   // fp32 path
      g.out16 = ab;    // bf16 path
      g.out_ustride = ss;
      g.ldo = (int32_t)sp;
      tr.before(MUON_KERNEL_GRAM);
      launch_phase<GRAM>(bf16, T, c.tall ? 3 : 0, g, ca, s);
      tr.after_ns(MUON_KERNEL_GRAM, c);
      // Polynomial: B' = a*I + b*A + c*A*A (A symmetric: both operands
      // K-contiguous; a*I carries the apply's a*X term).
      std::memset(&g, 0, sizeof(g));
      g.n_units = U;
      g.flag = flag;
      g.a = aop;
      g.b = aop;
      g.a_ustride = g.b_ustride = ss;
      g.lda = g.ldb = (int32_t)sp;
      g.M = g.N = g.K = (int32_t)sp;
      g.tiles_m = g.tiles_n = (int32_t)(sp / T);
      g.sym = 1;       // B' is symmetric as well
      g.out32 = bf16 ? nullptr : static_cast<float*>(bop);
      g.out16 = bf16 ? bop : nullptr;
      g.out_ustride = ss;
      g.ldo = (int32_t)sp;
      g.aux = a32;
      g.aux16 = ab;
      g.aux_ustride = ss;
      g.ldaux = (int32_t)sp;
      g.ca = sg.a;
      g.cb = sg.b;
      g.cc = sg.c;
      tr.before(MUON_KERNEL_POLY);
      launch_phase<POLY>(bf16, T, 0, g, ca, s);
      tr.after_ns(MUON_KERNEL_POLY, c);
      // Apply: X' = B'*X (wide) or X*B' (tall).
      std::memset(&g, 0, sizeof(g));
      g.n_units = U;
      g.flag = flag;
      g.M = (int32_t)c.rows_pad;
      g.N = (int32_t)c.cols_pad;
      g.K = (int32_t)sp;
      g.tiles_m = (int32_t)(c.rows_pad / T);
      g.tiles_n = (int32_t)(c.cols_pad / T);
      if (!c.tall) {
        g.a = bop;           // B[m][k]
        g.a_ustride = ss;
        g.lda = (int32_t)sp;
        g.b = bf16 ? xop[cur] : xt[cur];  // X[k][n]: K-major (bf16) or rows of X^T
        g.b_ustride = xs;
        g.ldb = (int32_t)(bf16 ? c.cols_pad : c.rows_pad);
      } else {
        g.a = xop[cur];      // X[m][k]
        g.a_ustride = xs;
        g.lda = (int32_t)c.cols_pad;
        g.b = bop;           // B[k][n] = B[n][k] (symmetric)
        g.b_ustride = ss;
        g.ldb = (int32_t)sp;
      }
      g.out32 = bf16 ? nullptr : x32[nxt];
      g.out16 = bf16 ? (void*)xb[nxt] : nullptr;
      g.out_ustride = xs;
      g.ldo = (int32_t)c.cols_pad;
      g.outt = xt[nxt];
      g.ldt = (int32_t)c.rows_pad;
      g.fold = it == 0 ? fold_scale : nullptr;
      g.final_mode = last ? (step ? FINAL_STEP : FINAL_NSOUT) : FINAL_NONE;
      tr.before(MUON_KERNEL_APPLY);
      launch_phase<APPLY>(bf16, T, c.tall ? 0 : 2, g, ca, s);
      tr.after_ns(MUON_KERNEL_APPLY, c);
    }
  }
  if (hipGetLastError() != hipSuccess) return MUON_ERR_HIP;
  return MUON_OK;
}

// scratch_ws: instead of a caller workspace, the library's fixed device
// scratch (muon_step_batched_noalloc); ws and ws_bytes are then ignored.
int scratch_workspace(void** ws, size_t* bytes);

int run(bool step, float* const* outs, const void* const* ins, float* const* moms,
        const muon_matrix_desc* mats, int64_t n, const muon_hyper* h, void* ws, size_t ws_bytes,
        hipStream_t stream, muon_trace* trace, bool scratch_ws = false) {
  try {
    int st = validate_hyper(h);
    if (st != MUON_OK) return st;
    st = validate_descs(mats, n, step);
    if (st != MUON_OK) return st;
    if (n == 0) return MUON_OK;
    if (!outs || !ins || (step && !moms)) return MUON_ERR_NULL;
    std::vector<Range> written, read;
    for (int64_t i = 0; i < n; ++i) {
      const muon_matrix_desc& d = mats[i];
      if (!outs[i] || !ins[i] || (step && !moms[i])) return MUON_ERR_NULL;
      if (misaligned(outs[i]) || misaligned(ins[i]) || (step && misaligned(moms[i])))
        return MUON_ERR_ALIGN;
      const uintptr_t elems = (uintptr_t)(d.batch * d.rows * d.cols);
      const uintptr_t gsz = (step && d.grad_dtype == MUON_DTYPE_BF16) ? 2 : 4;
      written.push_back({(uintptr_t)outs[i], (uintptr_t)outs[i] + elems * 4, (int)i});
      if (step) {
        written.push_back({(uintptr_t)moms[i], (uintptr_t)moms[i] + elems * 4, (int)i});
        read.push_back({(uintptr_t)ins[i], (uintptr_t)ins[i] + elems * gsz, -1 - (int)i});
      } else {
        // NS only: the input may be the bank's own output buffer, exactly.
        read.push_back({(uintptr_t)ins[i], (uintptr_t)ins[i] + elems * 4, (int)i});
      }
    }
    st = check_alias(written, read);
    if (st != MUON_OK) return st;
    std::vector<Chunk> chunks;
    st = plan(mats, n, h, step, &chunks);
    if (st != MUON_OK) return st;
    const size_t need = workspace_of(chunks, h, !scratch_ws);
    if (scratch_ws) {
      // the fixed scratch: refuse a step that needs more, before anything runs
      if (need > kScratchBytes) return MUON_ERR_WORKSPACE;
      st = scratch_workspace(&ws, &ws_bytes);
      if (st != MUON_OK) return st;
    }
    if (need > 0 && (!ws || ws_bytes < need)) return MUON_ERR_WORKSPACE;
    if (((uintptr_t)ws & (kAlign - 1)) != 0) return MUON_ERR_ALIGN;
    Tracer tr{trace, stream};
    if (trace) trace->count = 0;
    // The scratch's status header cannot be read by the callers of the
    // scratch entry point, so their passes run as one launch per product,
    // whose kernels never wait (bit-identical to the persistent launch).
    const bool allow_waits = !scratch_ws;
    // Riding passes that run inside their stacked pass's launch on this
    // device: the stacked pass takes one claim queue there.
    std::vector<char> rides(chunks.size(), 0);
    if (allow_waits) {
      int total = 0;
      for (int i = 0; i < h->n_stages; ++i) total += h->stages[i].steps;
      for (const Chunk& c : chunks) {
        if (c.rider < 0) continue;
        DeviceInfo di;
        st = device_info(&di);
        if (st != MUON_OK) return st;
        const Chunk& r = chunks[(size_t)c.rider];
        if (queues_for(c.n_units, di.xccs) == 1 &&
            persistent_items(c, total) + persistent_items(r, total) < INT32_MAX / 2)
          rides[(size_t)c.rider] = 1;
      }
    }
    bool first = true;
    for (size_t i = 0; i < chunks.size(); ++i) {
      if (rides[i]) continue;
      const Chunk& c = chunks[i];
      const Chunk* rider = c.rider >= 0 && rides[(size_t)c.rider] ? &chunks[(size_t)c.rider] : nullptr;
      st = run_chunk(c, h, step, outs, ins, moms, mats, static_cast<unsigned char*>(ws), stream, tr,
                     first, allow_waits, rider);
      if (st != MUON_OK) return st;
      first = false;
    }
    return MUON_OK;
  } catch (const std::bad_alloc&) {
    return MUON_ERR_SHAPE;
  } catch (...) {
    return MUON_ERR_HIP;
  }
}

}  // namespace

extern "C" {

void muon_hyper_default(muon_hyper* h) {
  if (!h) return;
  std::memset(h, 0, sizeof(*h));
  h->lr = 2.7e-4f;
  h->mu = 0.95f;
  h->weight_decay = 0.1f;
  h->gamma = 0.18f;
  h->scale_mode = MUON_SCALE_SPECTRAL;
  h->ns_precision = MUON_NS_BF16;
  h->batch_update_size = 0;
  h->schedule = MUON_SCHEDULE_AUTO;
  h->nesterov_style = MUON_NESTEROV_SGD;
  h->step = 1;
  h->n_stages = 2;
  h->stages[0] = {8, 3.4445f, -4.7750f, 2.0315f};
  h->stages[1] = {2, 2.0f, -1.5f, 0.5f};
}

int muon_workspace_size(const muon_matrix_desc* mats, int64_t n, const muon_hyper* h,
                        size_t* bytes) {
  try {
    if (!bytes) return MUON_ERR_NULL;
    int st = validate_hyper(h);
    if (st != MUON_OK) return st;
    st = validate_descs(mats, n, false);
    if (st != MUON_OK) return st;
    std::vector<Chunk> chunks;
    st = plan(mats, n, h, true, &chunks);
    if (st != MUON_OK) return st;
    // Step and NS-only group the same units when dtypes agree; take the
    // larger of the two plans so that one size serves both.
    std::vector<Chunk> chunks_ns;
    st = plan(mats, n, h, false, &chunks_ns);
    if (st != MUON_OK) return st;
    *bytes = std::max(workspace_of(chunks, h), workspace_of(chunks_ns, h));
    return MUON_OK;
  } catch (...) {
    return MUON_ERR_SHAPE;
  }
}

int muon_step_batched_traced(float* const* params, const void* const* grads, float* const* momenta,
                             const muon_matrix_desc* mats, int64_t n, const muon_hyper* h,
                             void* workspace, size_t workspace_bytes, hipStream_t stream,
                             muon_trace* trace) {
  return run(true, params, grads, momenta, mats, n, h, workspace, workspace_bytes, stream, trace);
}

int muon_step_batched(float* const* params, const void* const* grads, float* const* momenta,
                      const muon_matrix_desc* mats, int64_t n, const muon_hyper* h,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run(true, params, grads, momenta, mats, n, h, workspace, workspace_bytes, stream, nullptr);
}

int muon_step_batched_noalloc(float* const* params, const void* const* grads,
                              float* const* momenta, const muon_matrix_desc* mats, int64_t n,
                              const muon_hyper* h, hipStream_t stream) {
  return run(true, params, grads, momenta, mats, n, h, nullptr, 0, stream, nullptr, true);
}

int muon_newton_schulz_batched_traced(const float* const* x_in, float* const* o_out,
                                      const muon_matrix_desc* mats, int64_t n, const muon_hyper* h,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream,
                                      muon_trace* trace) {
  return run(false, o_out, reinterpret_cast<const void* const*>(x_in), nullptr, mats, n, h,
             workspace, workspace_bytes, stream, trace);
}

int muon_newton_schulz_batched(const float* const* x_in, float* const* o_out,
                               const muon_matrix_desc* mats, int64_t n, const muon_hyper* h,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return muon_newton_schulz_batched_traced(x_in, o_out, mats, n, h, workspace, workspace_bytes,
                                           stream, nullptr);
}

const char* muon_status_string(int status) {
  switch (status) {
    case MUON_OK: return "ok";
    case MUON_ERR_NULL: return "a required pointer is NULL";
    case MUON_ERR_SHAPE: return "invalid shape (rows/cols/batch < 1, split_rows does not divide rows, or too large)";
    case MUON_ERR_DTYPE: return "unknown dtype, precision or scale mode";
    case MUON_ERR_ALIGN: return "a data pointer is not 16-byte aligned (workspace: 256-byte)";
    case MUON_ERR_WORKSPACE: return "workspace missing or smaller than muon_workspace_size()";
    case MUON_ERR_HYPER: return "invalid hyper-parameters";
    case MUON_ERR_HIP: return "HIP launch failed";
    case MUON_ERR_ALIAS: return "input and output buffers overlap";
    case MUON_ERR_SCHEDULE: return "an NS launch stopped: a wait on other workgroups ran out of time";
    default: return "unknown status";
  }
}

int muon_workspace_status(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!workspace) return MUON_ERR_NULL;
  if (workspace_bytes < kHeader) return MUON_ERR_WORKSPACE;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return MUON_ERR_ALIGN;
  // The header: stop flag of the last call, sticky flag of the calls
  // before it, and the marker of an initialised header (kernels.hpp).
  uint32_t words[4] = {0u, 0u, 0u, 0u};
  if (hipMemcpyAsync(words, workspace, sizeof(words), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return MUON_ERR_HIP;
  uint64_t magic = 0;
  std::memcpy(&magic, words + 2, sizeof(magic));
  if (magic != kStatusMagic) return MUON_OK;  // no call has used this workspace yet
  if ((words[0] | words[1]) == 0u) return MUON_OK;
  // Reported once: clear both flags before returning.
  if (hipMemsetAsync(workspace, 0, 2 * sizeof(uint32_t), stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return MUON_ERR_HIP;
  return MUON_ERR_SCHEDULE;
}

int muon_abi_version(void) { return 6; }

}  // extern "C"
