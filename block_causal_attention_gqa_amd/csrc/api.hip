// Host side of the C ABI declared in include/bc.h: argument validation,
// workspace sizing, the split plan of the attention, and kernel launches.
// Nothing here allocates device memory or keeps state between calls.

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

#include "bc_internal.h"

namespace {

using namespace bc;

bool dtype_ok(int d) { return d == BC_F32 || d == BC_BF16; }
int elem_bytes(int d) { return d == BC_BF16 ? 2 : 4; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int check_cache(const bc_kv_cache* c) {
  if (!c || !c->k || !c->v) return BC_ERR_ARG;
  if (!dtype_ok(c->dtype)) return BC_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return BC_ERR_UNSUPPORTED;
  if (c->n_seq < 1 || c->n_kv_heads < 1 || c->capacity < 1) return BC_ERR_ARG;
  return BC_OK;
}

int check_blk_off(const int32_t* off, int n_blk, int n_rows, int max_rows_per_block) {
  if (!off) return BC_ERR_ARG;
  if (n_blk < 1) return BC_ERR_ARG;
  if (n_blk > BC_MAX_BLOCKS) return BC_ERR_UNSUPPORTED;
  if (off[0] != 0 || off[n_blk] != n_rows) return BC_ERR_ARG;
  for (int b = 0; b < n_blk; ++b) {
    if (off[b + 1] <= off[b]) return BC_ERR_ARG;
    if (off[b + 1] - off[b] > max_rows_per_block) return BC_ERR_UNSUPPORTED;
  }
  return BC_OK;
}

// ------------------------------------------------------------ attention plan
struct Plan {
  int waves, cols, fork_rows, direct, P, n_mt_prefix, n_mt_active, n_prefix_items, n_items, rows_total, n_slots;
  int xmap, tile_rows, unit_tiles, n_units, units_per_xcd;
  bool compact;        // compact split partials (bf16 inputs, many rows)
  bool fold;           // active keys in the last prefix chunk's items (no slot P)
  size_t o_bytes, ml_bytes, total_bytes;   // what this call's plan writes
  size_t reserve_bytes;   // what bc_attn_workspace_bytes reports: at least total_bytes
};

int validate_attn(const bc_kv_cache* prefix, const bc_kv_cache* priv, const bc_active* a,
                  int32_t n_splits) {
  int st = check_cache(prefix);
  if (st) return st;
  if (!a || !a->q || !a->k || !a->v) return BC_ERR_ARG;
  if (a->n_seq < 1 || a->n_rows < 1 || a->n_q_heads < 1) return BC_ERR_ARG;
  if (a->n_seq > BC_MAX_SEQ) return BC_ERR_UNSUPPORTED;
  if (a->n_q_heads % prefix->n_kv_heads) return BC_ERR_ARG;
  if ((st = check_blk_off(a->blk_off, a->n_blk, a->n_rows, 1 << 30))) return st;
  if (n_splits < 0 || n_splits > 256) return BC_ERR_ARG;
  if (priv) {
    if ((st = check_cache(priv))) return st;
    if (prefix->n_seq != 1 || priv->n_seq != a->n_seq) return BC_ERR_ARG;
    if (priv->dtype != prefix->dtype) return BC_ERR_UNSUPPORTED;
    if (priv->n_kv_heads != prefix->n_kv_heads || priv->head_dim != prefix->head_dim) return BC_ERR_ARG;
  } else if (prefix->n_seq != a->n_seq) {
    return BC_ERR_ARG;
  }
  // all offsets of the kernels are 64-bit; keep the row/item counts in int range
  const long long rows = (long long)a->n_seq * a->n_rows * a->n_q_heads;
  if (rows > (1LL << 26)) return BC_ERR_UNSUPPORTED;
  return BC_OK;
}

// Prefix split count P when the caller leaves it to the library.  A
// launch's time is modelled as
//   max(rounds * (tiles per item * t_tile + t_item), kv_bytes / bw + t_item)
//   + (P + 1) * t_slot
// with rounds = ceil(items / co-resident workgroups): splitting the prefix
// shortens every item but adds a partial slot per output row that the
// combine writes and reads back, and no split count beats streaming the
// K/V bytes from HBM once.  Constants measured on MI355X: ~1.9 us per
// 64-key tile with one workgroup per CU and ~2.5 us with two (512
// co-resident), ~2 us of fixed cost per item (Q load, first tile, partial
// write), K/V and partial slots streamed at ~5 TB/s.
// partial workgroups resident at once: two per CU on 256 CUs
constexpr int kSlotsResident = 512;

int auto_splits(int row_tiles, int maxlen, double kv_bytes, int rows_total, double slot_row_bytes, bool wide,
                int max_splits = 256) {
  constexpr int kCUs = 256;
  constexpr double kTileUs1 = 1.9, kTileUs2 = 2.5, kItemUs = 2.0, kBytesPerUs = 5.0e6;
  // Slot traffic of two-column-tile calls (many rows, long items) is priced
  // at an effective ~2 TB/s, fitted to forced split sweeps: the fork at
  // N = 16 was 28.4-29.1 us at P = 6 against 30.5-32 us at P = 9 (this
  // model picks 5: 29.2-30.1 us), the large-block batch 16 best at P = 2.
  // One-column-tile calls (bs1) are launch-bound and keep 5 TB/s, where
  // P ~ 25 is the measured optimum.
  const double slot_us = (double)rows_total * slot_row_bytes * 2.0 / (wide ? 2.0e6 : kBytesPerUs);
  const double floor_us = kv_bytes / kBytesPerUs + kItemUs;
  const int most = std::max(1, std::min(max_splits, (maxlen + kAttnKeyTile - 1) / kAttnKeyTile));
  int best = 1;
  double best_us = 1e300;
  for (int P = 1; P <= most; ++P) {
    const int per = (maxlen + P - 1) / P;
    const int tiles = std::max(1, (per + kAttnKeyTile - 1) / kAttnKeyTile);
    const long long items = (long long)row_tiles * P;
    const long long rounds = (items + kSlotsResident - 1) / kSlotsResident;
    const double tile_us = items <= kCUs ? kTileUs1 : kTileUs2;
    const double us = std::max(rounds * (tiles * tile_us + kItemUs), floor_us) + (P + 1) * slot_us;
    if (us < best_us - 1e-9) { best_us = us; best = P; }
  }
  return best;
}

// lengths[s] are the prefix lengths the plan is made for (the capacities when
// sizing the workspace: the plan is monotone in the lengths, so that bound
// covers every call with the same shapes).
void make_plan(const bc_kv_cache* prefix, const bc_kv_cache* priv, const bc_active* a,
               const int* lengths, int32_t n_splits, Plan* p, int* chunk) {
  const int S = a->n_seq, R = a->n_rows, Hq = a->n_q_heads, Hkv = prefix->n_kv_heads;
  const int group = Hq / Hkv, D = prefix->head_dim;
  const bool fork = priv != nullptr;
  // Split partials: compact (int16 output, 16-byte record) for bf16 inputs
  // with many output rows, where their write and read-back is a large part
  // of the call; float32 otherwise.  The extra quantising work sits on every
  // workgroup's tail, which a latency-bound call with few rows pays for
  // (measured: +4% at 512 rows, -14% at 1536 rows over a 3282-key prefix).
  // The choice depends on the shapes only, so the workspace size a call
  // needs never exceeds the size at full capacity.
  const bool compact = prefix->dtype == BC_BF16 && S * R * Hq >= kCompactRows;
  p->compact = compact;
  const double slot_row_bytes = compact ? D * 2.0 + 16.0 : D * 4.0 + 8.0;
  const int groups = fork ? Hkv : S * Hkv;
  const int rows_group = fork ? S * R * group : R * group;
  int maxlen = 0;
  for (int s = 0; s < prefix->n_seq; ++s) maxlen = std::max(maxlen, lengths[s]);
  // K/V bytes of the prefix as streamed from HBM (a shared fork prefix once)
  double kv = 0;
  for (int s = 0; s < prefix->n_seq; ++s) kv += (double)lengths[s] * Hkv * D * 2.0 * elem_bytes(prefix->dtype);
  // Row tiles of 128 rows (4 waves x 32), or of 64 rows: bf16 as 4 waves x
  // 16 rows, which also halves each wave's per-tile dependency chain; fp32
  // as 2 waves x 32.  The 128-row form needs two of its workgroups on a CU
  // (one wave per SIMD cannot hide its own latencies), so when its prefix
  // items would give each CU at most one -- few row tiles, or few splits --
  // the 64-row form, with twice the items, is used.  Measured (call times):
  // large-block batch 16 38.7 -> 36.8 us and batch 8 27.0 -> 25.1 us (256
  // items with 128-row tiles); fork N = 16 29.4 -> 26.1 us (240); fork
  // N = 32 / 48 / 64 (480 / 432 / 384 items) are faster with 128 rows.
  // Groups of at most 64 rows also take 64-row tiles: a 128-row tile would
  // be at least half padding, whose MFMAs and operand reads every wave still
  // issues (measured, large-block batch 16 over a 2176-key prefix, block
  // sizes 1 / 4 / 8 / 16: call 28.9 / 31.1 / 31.4 / 33.5 -> 26.4 / 28.4 /
  // 28.9 / 30.3 us back to back).
  bool small = groups * ((rows_group + 127) / 128) < 32 || rows_group <= 64;
  int P = n_splits;
  if (!small && prefix->dtype == BC_BF16) {
    const int mt2 = (rows_group + 127) / 128;
    const int P2 = P ? P : auto_splits(groups * mt2, maxlen, kv, S * R * Hq, slot_row_bytes, true);
    small = (long long)groups * mt2 * P2 <= 256;
  }
  if (prefix->dtype == BC_BF16) { p->waves = 4; p->cols = small ? 1 : 2; }
  else { p->waves = small ? 2 : 4; p->cols = 2; }
  const int tile_rows = p->waves * p->cols * 16;
  p->n_mt_prefix = (rows_group + tile_rows - 1) / tile_rows;
  p->n_mt_active = (R * group + tile_rows - 1) / tile_rows;
  if (P == 0) {
    // Without a fork and with at most 8 row tiles, the XCD-aligned mapping
    // (below) puts each row tile's P + 1 items on an XCD of its own.  Past
    // its 32 CUs they double up, and for these latency-bound one-column-tile
    // items a second workgroup on a CU costs more than the longer items of
    // fewer splits (measured, bs1 section decode: 12 rows over 3072 keys 10.1
    // us with the model's 48 one-tile splits against 8.5 us at 24-30 two-tile
    // splits; 6 rows over 3276 / 3346 keys 9.3 against 8.2-8.4 us; the decode
    // 1567 -> 1538 us), so the split count keeps them on a CU each.  (With
    // more row tiles per XCD the model's trade stays: capping those measured
    // slower.)
    int max_splits = 256;
    const int row_tiles = groups * p->n_mt_prefix;
    if (!fork && p->cols == 1 && row_tiles <= 8) max_splits = 31;
    P = auto_splits(row_tiles, maxlen, kv, S * R * Hq, slot_row_bytes, p->cols == 2, max_splits);
  }
  p->P = P;
  p->n_prefix_items = groups * P * p->n_mt_prefix;
  const int n_active_items = S * Hkv * p->n_mt_active;
  // Fold: without a fork, when the prefix items fill at most the co-resident
  // workgroups (two per CU) but the active items would not fit beside them,
  // the active items would run as a second round behind the longest prefix
  // item.  Then the last prefix chunk of each row tile also takes its active
  // keys instead (the chunks are cut so that it stays no longer than the
  // others): one round, one slot fewer to write and merge.  Measured on the
  // large-block batch 16 (512 prefix items of 17 tiles, 256 active items):
  // call 40.3 -> 38.5 us with the caches rotated, 35.6 -> 34.9 us back to
  // back.  Calls whose active items fit in the first round (bs1) keep them
  // apart: there folding only lengthens the slowest item (measured: decode
  // 177K -> 173K tok/s).
  p->fold = !fork && p->n_prefix_items <= kSlotsResident && p->n_prefix_items + n_active_items > kSlotsResident;
  const int act = p->fold ? R : 0;   // keys the last chunk also takes
  for (int s = 0; s < prefix->n_seq; ++s) {
    const int per = (lengths[s] + act + P - 1) / P;
    chunk[s] = std::max(kAttnKeyTile, (per + kAttnKeyTile - 1) / kAttnKeyTile * kAttnKeyTile);
  }
  p->n_slots = p->fold ? P : P + 1;
  p->n_items = p->n_prefix_items + (p->fold ? 0 : n_active_items);
  // Without a fork every row of a row tile gets its records from that tile's
  // items, so the tile, its splits and the combine of its rows can share an
  // XCD (measured: a kernel reading 6.8 MB that the previous kernel wrote
  // on other XCDs took 3.4 us longer than reading what its own XCD wrote).
  // With a fork the prefix row tiles span rollouts while the active items
  // tile each rollout's rows, so the fork keeps the key-chunk mapping.  The
  // placement (workgroup id mod 8) holds for workgroups dispatched while the
  // GPU has room for them; with more workgroups than are resident at once
  // (two per CU) the later ones land wherever a CU frees up, so larger grids
  // keep the key-chunk mapping too (measured: large-block batch 16, 768
  // workgroups, 36.6 -> 49.4 us with the aligned mapping; bs1, 208, 10.7 ->
  // 9.8 us).
  p->tile_rows = tile_rows;
  p->unit_tiles = groups >= 8 ? p->n_mt_prefix : 1;
  p->n_units = groups >= 8 ? groups : groups * p->n_mt_prefix;
  p->units_per_xcd = (p->n_units + 7) / 8;
  p->xmap = !fork && 8LL * p->units_per_xcd * p->unit_tiles * p->n_slots < 512;
  p->rows_total = S * R * Hq;
  // sized for P + 1 slots whether or not the call folds, so that a
  // workspace sized at full capacity holds every call with these shapes
  p->o_bytes = align256((size_t)(P + 1) * p->rows_total * D * (compact ? 2 : 4));
  p->ml_bytes = align256((size_t)(P + 1) * p->rows_total * (compact ? 16 : 8));
  p->total_bytes = p->o_bytes + p->ml_bytes;
  p->reserve_bytes = p->total_bytes;
  p->fork_rows = 0;
  p->direct = 0;
  // Fork, row-tile form: when half of a rollout's rows per KV head fill more
  // than half of one 96-row tile (bf16, head_dim 128), each (KV head,
  // rollout, half) row tile takes P_r key splits, as many as give every CU
  // one workgroup (2 N Hkv P_r >= 256) while each split keeps at least 12
  // key tiles; a workgroup covers its split's prefix chunk -- the last also the
  // rollout's private keys and the active keys, so there is no slot for
  // them -- in two key halves merged in LDS (attn_fork_rows_kernel).  With
  // P_r = 1 (N >= 128 / Hkv) it writes the output itself and the combine
  // does nothing.  Emptier tiles would pay a full tile's MFMAs for a few
  // rows; fewer workgroups than CUs, or shorter splits (small N), keep the
  // split plan (measured at N = 4: 16 splits of 3 tiles, 14.8 -> 16.2 us;
  // N = 16, 4 splits of 13 tiles: 26.2 -> 25.2 us; N = 64, one split: 63 ->
  // 58 us, draft passes over a 3282-key prefix).  The
  // workspace size reported is the larger of the two plans', so that a
  // workspace sized at capacity serves every call with these shapes.
  // (Without a fork the same form, 64-row tiles of half a sequence's rows,
  // measured no better on the large-block batch 16 call: 33.4 -> 32.7 us
  // back to back, 39.8 -> 41.9 us after a clean flush.)
  const int half_rows = (R * group + 1) / 2;
  if (fork && prefix->dtype == BC_BF16 && D == 128 && n_splits == 0 && half_rows <= kForkTileRows &&
      2 * half_rows > kForkTileRows) {
    const int tiles = S * Hkv * 2;
    const int Pr = std::max(1, std::min(256 / tiles, maxlen / (12 * kAttnKeyTile)));
    if ((long long)tiles * Pr >= 256) {
      p->fork_rows = 1;
      p->direct = Pr == 1;
      p->P = Pr;
      p->n_slots = Pr;
      const int per = (maxlen + Pr - 1) / Pr;
      chunk[0] = std::max(kAttnKeyTile, (per + kAttnKeyTile - 1) / kAttnKeyTile * kAttnKeyTile);
      p->o_bytes = align256((size_t)Pr * p->rows_total * D * (compact ? 2 : 4));
      p->ml_bytes = align256((size_t)Pr * p->rows_total * (compact ? 16 : 8));
      p->total_bytes = p->o_bytes + p->ml_bytes;
      p->reserve_bytes = std::max(p->reserve_bytes, p->total_bytes);
    }
  }
}

}  // namespace

extern "C" {

const char* bc_status_str(int status) {
  switch (status) {
    case BC_OK: return "BC_OK";
    case BC_ERR_ARG: return "BC_ERR_ARG: malformed argument";
    case BC_ERR_UNSUPPORTED: return "BC_ERR_UNSUPPORTED: outside what the kernels handle";
    case BC_ERR_CAPACITY: return "BC_ERR_CAPACITY: commit past the cache capacity";
    case BC_ERR_ORDER: return "BC_ERR_ORDER: commit does not start at the current length";
    case BC_ERR_WORKSPACE: return "BC_ERR_WORKSPACE: workspace missing or too small";
    case BC_ERR_HIP: return "BC_ERR_HIP: the HIP runtime rejected a launch";
    case BC_ERR_SCRATCH:
      return "BC_ERR_SCRATCH: the call needs more than the static scratch (BC_STATIC_SCRATCH_BYTES) holds";
    case BC_ERR_CALLBACK: return "BC_ERR_CALLBACK: a caller callback returned nonzero";
    default: return "unknown bc_status";
  }
}

int bc_kv_commit(const bc_kv_cache* cache, int32_t* len, int32_t seq, int32_t start, int32_t n_rows,
                 const void* blk_k, const void* blk_v, void* stream) {
  int st = check_cache(cache);
  if (st) return st;
  if (!len || !blk_k || !blk_v) return BC_ERR_ARG;
  const bool all = seq == BC_ALL_SEQ;
  if ((!all && (seq < 0 || seq >= cache->n_seq)) || n_rows < 1) return BC_ERR_ARG;
  const int s0 = all ? 0 : seq, n_seq = all ? cache->n_seq : 1;
  for (int s = s0; s < s0 + n_seq; ++s)
    if (start != len[s]) return BC_ERR_ORDER;
  if ((long long)start + n_rows > cache->capacity) return BC_ERR_CAPACITY;
  const int D = cache->head_dim, Hkv = cache->n_kv_heads, eb = elem_bytes(cache->dtype);
  const long long head_stride = (long long)cache->capacity * D;
  const long long seq_stride = head_stride * Hkv;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  // sequences are consecutive runs of Hkv heads at the same head stride, so
  // a commit of every sequence is one copy over n_seq * Hkv heads
  char* kdst = static_cast<char*>(cache->k) + s0 * seq_stride * eb;
  char* vdst = static_cast<char*>(cache->v) + s0 * seq_stride * eb;
  if (launch_commit(kdst, vdst, blk_k, blk_v, cache->dtype, n_seq * Hkv, D, head_stride, start, n_rows, strm) !=
      hipSuccess)
    return BC_ERR_HIP;
  for (int s = s0; s < s0 + n_seq; ++s) len[s] = start + n_rows;
  return BC_OK;
}

size_t bc_attn_workspace_bytes(const bc_kv_cache* prefix, const bc_kv_cache* priv, const bc_active* a,
                               int32_t n_prefix_splits) {
  if (validate_attn(prefix, priv, a, n_prefix_splits) != BC_OK) return 0;
  int caps[BC_MAX_SEQ];
  for (int s = 0; s < prefix->n_seq; ++s) caps[s] = prefix->capacity;
  Plan p;
  int chunk[BC_MAX_SEQ];
  make_plan(prefix, priv, a, caps, n_prefix_splits, &p, chunk);
  return p.reserve_bytes;
}

}  // extern "C"

namespace {

// Every check of an attention call's arguments except the workspace.
int validate_attn_call(const bc_kv_cache* prefix, const int32_t* prefix_len, const bc_kv_cache* priv,
                       const int32_t* priv_len, const bc_active* a, int32_t mask, float scale,
                       int32_t n_prefix_splits, const void* out) {
  int st = validate_attn(prefix, priv, a, n_prefix_splits);
  if (st) return st;
  if (!prefix_len || !out || (priv && !priv_len)) return BC_ERR_ARG;
  if (mask != BC_MASK_BLOCK_BIDIR && mask != BC_MASK_BLOCK_CAUSAL) return BC_ERR_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return BC_ERR_ARG;
  for (int s = 0; s < prefix->n_seq; ++s)
    if (prefix_len[s] < 0 || prefix_len[s] > prefix->capacity) return BC_ERR_ARG;
  if (priv)
    for (int s = 0; s < a->n_seq; ++s)
      if (priv_len[s] < 0 || priv_len[s] > priv->capacity) return BC_ERR_ARG;
  return BC_OK;
}

// Validate an attention call and fill the kernel arguments; BC_OK or an error.
int prepare_attn(const bc_kv_cache* prefix, const int32_t* prefix_len, const bc_kv_cache* priv,
                 const int32_t* priv_len, const bc_active* a, int32_t mask, float scale, int32_t n_prefix_splits,
                 void* out, void* ws, size_t ws_bytes, AttnArgs* args) {
  int st = validate_attn_call(prefix, prefix_len, priv, priv_len, a, mask, scale, n_prefix_splits, out);
  if (st) return st;

  std::memset(args, 0, sizeof(*args));
  if (!ws) return BC_ERR_WORKSPACE;
  Plan p;
  make_plan(prefix, priv, a, prefix_len, n_prefix_splits, &p, args->chunk);
  if (ws_bytes < p.total_bytes) {
    // An explicit split count must fit.  An automatic one is reduced to
    // what the workspace holds (a workspace sized by bc_attn_workspace_bytes
    // always holds at least the split count chosen at full capacity).
    if (n_prefix_splits > 0) return BC_ERR_WORKSPACE;
    int P = p.P;
    while (P > 1 && ws_bytes < p.total_bytes) {
      --P;
      make_plan(prefix, priv, a, prefix_len, P, &p, args->chunk);
    }
    if (ws_bytes < p.total_bytes) return BC_ERR_WORKSPACE;
  }
  const int D = prefix->head_dim;
  args->q = a->q;
  args->out = out;
  args->pk = prefix->k;
  args->pv = prefix->v;
  args->p_head_stride = (long long)prefix->capacity * D;
  args->p_seq_stride = args->p_head_stride * prefix->n_kv_heads;
  if (priv) {
    args->vk = priv->k;
    args->vv = priv->v;
    args->v_head_stride = (long long)priv->capacity * D;
    args->v_seq_stride = args->v_head_stride * priv->n_kv_heads;
  }
  args->ak = a->k;
  args->av = a->v;
  args->ws_o = ws;
  args->ws_ml = static_cast<char*>(ws) + p.o_bytes;
  args->compact = p.compact ? 1 : 0;
  args->scale_log2 = scale * 1.4426950408889634f;
  args->S = a->n_seq;
  args->R = a->n_rows;
  args->Hq = a->n_q_heads;
  args->Hkv = prefix->n_kv_heads;
  args->group = a->n_q_heads / prefix->n_kv_heads;
  args->D = D;
  args->waves = p.waves;
  args->cols = p.cols;
  args->fork_rows = p.fork_rows;
  args->direct = p.direct;
  args->fork = priv ? 1 : 0;
  args->causal = mask == BC_MASK_BLOCK_CAUSAL;
  args->n_splits = p.P;
  args->n_slots = p.n_slots;
  args->fold = p.fold ? 1 : 0;
  args->n_mt_prefix = p.n_mt_prefix;
  args->n_mt_active = p.n_mt_active;
  args->n_prefix_items = p.n_prefix_items;
  args->n_items = p.n_items;
  args->rows_total = p.rows_total;
  args->n_blk = a->n_blk;
  for (int b = 0; b <= a->n_blk; ++b) args->blk_off[b] = a->blk_off[b];
  for (int s = 0; s < prefix->n_seq; ++s) args->prefix_len[s] = prefix_len[s];
  if (priv)
    for (int s = 0; s < a->n_seq; ++s) args->priv_len[s] = priv_len[s];
  // every divisor is >= 1 and every dividend below 2^31 (rows < 2^26)
  args->dv_mt_prefix = make_fastdiv(p.n_mt_prefix);
  args->dv_splits = make_fastdiv(p.P);
  args->dv_hkv = make_fastdiv(args->Hkv);
  args->dv_mt_active = make_fastdiv(p.n_mt_active);
  args->dv_rows = make_fastdiv(args->R * args->group);
  args->dv_group = make_fastdiv(args->group);
  args->xmap = p.xmap;
  args->tile_rows = p.tile_rows;
  args->unit_tiles = p.unit_tiles;
  args->n_units = p.n_units;
  args->units_per_xcd = p.units_per_xcd;
  args->dv_slots = make_fastdiv(p.n_slots);
  args->dv_unit_tiles = make_fastdiv(p.unit_tiles);
  return BC_OK;
}

int validate_unmask(const float* logits, int32_t n_rows, int32_t vocab, const int32_t* blk_off, int32_t n_blk,
                    const int32_t* mode, const int32_t* n_div, float threshold, const uint8_t* masked,
                    const int32_t* tokens, const int32_t* n_commit, const void* ws, size_t ws_bytes) {
  if (!logits || !mode || !n_div || !masked || !tokens || !n_commit) return BC_ERR_ARG;
  if (n_rows < 1 || vocab < 1) return BC_ERR_ARG;
  if (n_rows > BC_MAX_SCAN_ROWS) return BC_ERR_UNSUPPORTED;
  int st = check_blk_off(blk_off, n_blk, n_rows, BC_MAX_BLOCK_ROWS);
  if (st) return st;
  for (int b = 0; b < n_blk; ++b) {
    if (mode[b] != BC_UNMASK_SEMI && mode[b] != BC_UNMASK_FULL) return BC_ERR_ARG;
    if (n_div[b] < 1) return BC_ERR_ARG;
  }
  if (!std::isfinite(threshold)) return BC_ERR_ARG;
  if (!ws || ws_bytes < bc_unmask_workspace_bytes(n_rows, vocab)) return BC_ERR_WORKSPACE;
  return BC_OK;
}

// Verify with the row tokens t_i = argmax(l_i * inv_t + g_i) (g null:
// argmax l_i).
int spec_verify(const float* logits, const float* noise, float inv_t, int32_t n_seq, int32_t n_lrows, int32_t vocab,
                const int32_t* draft, int32_t m, const uint8_t* fixed, const int32_t* first, int32_t* accept_len,
                int32_t* bonus, void* ws, size_t ws_bytes, void* stream) {
  if (!logits || !draft || !first || !accept_len || !bonus) return BC_ERR_ARG;
  if (n_seq < 1 || n_lrows < 1 || vocab < 1 || m < 1 || m > n_lrows) return BC_ERR_ARG;
  if ((long long)n_seq * n_lrows > BC_MAX_SCAN_ROWS) return BC_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < bc_verify_workspace_bytes(n_seq, n_lrows, vocab)) return BC_ERR_WORKSPACE;
  VerifyArgs args;
  std::memset(&args, 0, sizeof(args));
  args.logits = logits;
  args.noise = noise;
  args.inv_temperature = inv_t;
  args.n_seq = n_seq;
  args.n_lrows = n_lrows;
  args.vocab = vocab;
  args.n_chunks = scan_chunks(vocab);
  args.m = m;
  args.draft = draft;
  args.fixed = fixed;
  args.first = first;
  args.accept_len = accept_len;
  args.bonus = bonus;
  args.part = static_cast<ScanPartial*>(ws);
  (void)hipGetLastError();
  if (launch_verify(args, static_cast<hipStream_t>(stream)) != hipSuccess) return BC_ERR_HIP;
  return BC_OK;
}

void fill_unmask(const float* logits, int32_t n_rows, int32_t vocab, const int32_t* blk_off, int32_t n_blk,
                 const int32_t* mode, const int32_t* n_div, float threshold, uint8_t* masked, int32_t* tokens,
                 float* conf, int32_t* n_commit, void* ws, UnmaskArgs* args) {
  std::memset(args, 0, sizeof(*args));
  args->logits = logits;
  args->n_rows = n_rows;
  args->vocab = vocab;
  args->n_chunks = scan_chunks(vocab);
  args->n_blk = n_blk;
  args->masked = masked;
  args->tokens = tokens;
  args->conf = conf;
  args->n_commit = n_commit;
  args->part = static_cast<const ScanPartial*>(ws);
  args->threshold = threshold;
  for (int b = 0; b <= n_blk; ++b) args->blk_off[b] = blk_off[b];
  for (int b = 0; b < n_blk; ++b) {
    args->mode[b] = mode[b];
    args->n_div[b] = n_div[b];
  }
}

}  // namespace

namespace bc {
int prepare_attn_args(const bc_kv_cache* prefix, const int32_t* prefix_len, const bc_active* a, float scale,
                      void* out, void* ws, size_t ws_bytes, AttnArgs* args) {
  return prepare_attn(prefix, prefix_len, nullptr, nullptr, a, BC_MASK_BLOCK_BIDIR, scale, 0, out, ws, ws_bytes, args);
}
int prepare_unmask_args(const float* logits, int32_t n_rows, int32_t vocab, const int32_t* blk_off, int32_t n_blk,
                        const int32_t* mode, const int32_t* n_div, float threshold, uint8_t* masked, int32_t* tokens,
                        int32_t* n_commit, void* ws, size_t ws_bytes, UnmaskArgs* args) {
  const int st = validate_unmask(logits, n_rows, vocab, blk_off, n_blk, mode, n_div, threshold, masked, tokens,
                                 n_commit, ws, ws_bytes);
  if (st) return st;
  fill_unmask(logits, n_rows, vocab, blk_off, n_blk, mode, n_div, threshold, masked, tokens, nullptr, n_commit, ws,
              args);
  return BC_OK;
}
}  // namespace bc

extern "C" {

int bc_attn_partial(const bc_kv_cache* prefix, const int32_t* prefix_len, const bc_kv_cache* priv,
                    const int32_t* priv_len, const bc_active* a, int32_t mask, float scale, int32_t n_prefix_splits,
                    void* out, void* ws, size_t ws_bytes, void* stream) {
  AttnArgs args;
  const int st = prepare_attn(prefix, prefix_len, priv, priv_len, a, mask, scale, n_prefix_splits, out, ws,
                              ws_bytes, &args);
  if (st) return st;
  (void)hipGetLastError();
  return launch_attn_partial(args, prefix->dtype, static_cast<hipStream_t>(stream)) == hipSuccess ? BC_OK
                                                                                                   : BC_ERR_HIP;
}

int bc_attn_combine(const bc_kv_cache* prefix, const int32_t* prefix_len, const bc_kv_cache* priv,
                    const int32_t* priv_len, const bc_active* a, int32_t mask, float scale, int32_t n_prefix_splits,
                    void* out, void* ws, size_t ws_bytes, void* stream) {
  AttnArgs args;
  const int st = prepare_attn(prefix, prefix_len, priv, priv_len, a, mask, scale, n_prefix_splits, out, ws,
                              ws_bytes, &args);
  if (st) return st;
  (void)hipGetLastError();
  return launch_attn_combine(args, prefix->dtype, static_cast<hipStream_t>(stream)) == hipSuccess ? BC_OK
                                                                                                   : BC_ERR_HIP;
}

int bc_attn_step(const bc_kv_cache* prefix, const int32_t* prefix_len, const bc_kv_cache* priv,
                 const int32_t* priv_len, const bc_active* a, int32_t mask, float scale,
                 int32_t n_prefix_splits, void* out, void* ws, size_t ws_bytes, void* stream) {
  AttnArgs args;
  const int st = prepare_attn(prefix, prefix_len, priv, priv_len, a, mask, scale, n_prefix_splits, out, ws,
                              ws_bytes, &args);
  if (st) return st;
  (void)hipGetLastError();
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_attn_partial(args, prefix->dtype, s) != hipSuccess) return BC_ERR_HIP;
  if (launch_attn_combine(args, prefix->dtype, s) != hipSuccess) return BC_ERR_HIP;
  return BC_OK;
}

}  // extern "C"

// ------------------------------------------------- allocation-free attention
// The split partials of bc_attn_step_static live in this array.  In host code
// its name is only the host-side stand-in of the device variable: the device
// address comes from hipGetSymbolAddress, once per device, and only that
// address is ever handed to a kernel.
namespace {

static __device__ __align__(256) unsigned char scratch[BC_STATIC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxScratchDevices] = {};

// The current device's scratch address; BC_OK or an error.
int scratch_address(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return BC_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return BC_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BC_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return BC_OK;
}

}  // namespace

extern "C" {

int bc_attn_step_static(const bc_kv_cache* prefix, const int32_t* prefix_len, const bc_kv_cache* priv,
                        const int32_t* priv_len, const bc_active* a, int32_t mask, float scale,
                        int32_t n_prefix_splits, void* out, void* stream) {
  // validate before touching the device, so that bad arguments enqueue nothing
  int st = validate_attn_call(prefix, prefix_len, priv, priv_len, a, mask, scale, n_prefix_splits, out);
  if (st) return st;
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  AttnArgs args;
  st = prepare_attn(prefix, prefix_len, priv, priv_len, a, mask, scale, n_prefix_splits, out, ws,
                    BC_STATIC_SCRATCH_BYTES, &args);
  if (st == BC_ERR_WORKSPACE) return BC_ERR_SCRATCH;
  if (st) return st;
  (void)hipGetLastError();
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_attn_partial(args, prefix->dtype, s) != hipSuccess) return BC_ERR_HIP;
  if (launch_attn_combine(args, prefix->dtype, s) != hipSuccess) return BC_ERR_HIP;
  return BC_OK;
}

// unmask / verify workspaces hold the per-(row, chunk) scan partials.
size_t bc_unmask_workspace_bytes(int32_t n_rows, int32_t vocab) {
  if (n_rows < 1 || vocab < 1 || n_rows > BC_MAX_SCAN_ROWS) return 0;
  return align256((size_t)n_rows * scan_chunks(vocab) * sizeof(ScanPartial));
}

int bc_vocab_scan(const float* logits, int32_t n_rows, int32_t vocab, const uint8_t* row_mask, int32_t with_sum,
                  void* ws, size_t ws_bytes, void* stream) {
  if (!logits || n_rows < 1 || vocab < 1) return BC_ERR_ARG;
  if (n_rows > BC_MAX_SCAN_ROWS) return BC_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < bc_unmask_workspace_bytes(n_rows, vocab)) return BC_ERR_WORKSPACE;
  (void)hipGetLastError();
  return launch_scan(logits, n_rows, vocab, row_mask, with_sum != 0, static_cast<ScanPartial*>(ws),
                     static_cast<hipStream_t>(stream)) == hipSuccess ? BC_OK : BC_ERR_HIP;
}

int bc_unmask_decide(const float* logits, int32_t n_rows, int32_t vocab, const int32_t* blk_off, int32_t n_blk,
                     const int32_t* mode, const int32_t* n_div, float threshold, uint8_t* masked, int32_t* tokens,
                     float* conf, int32_t* n_commit, void* ws, size_t ws_bytes, void* stream) {
  const int st = validate_unmask(logits, n_rows, vocab, blk_off, n_blk, mode, n_div, threshold, masked, tokens,
                                 n_commit, ws, ws_bytes);
  if (st) return st;
  UnmaskArgs args;
  fill_unmask(logits, n_rows, vocab, blk_off, n_blk, mode, n_div, threshold, masked, tokens, conf, n_commit, ws,
              &args);
  (void)hipGetLastError();
  return launch_unmask_decide(args, static_cast<hipStream_t>(stream)) == hipSuccess ? BC_OK : BC_ERR_HIP;
}

int bc_unmask_select(const float* logits, int32_t n_rows, int32_t vocab, const int32_t* blk_off, int32_t n_blk,
                     const int32_t* mode, const int32_t* n_div, float threshold, uint8_t* masked, int32_t* tokens,
                     float* conf, int32_t* n_commit, void* ws, size_t ws_bytes, void* stream) {
  const int st = validate_unmask(logits, n_rows, vocab, blk_off, n_blk, mode, n_div, threshold, masked, tokens,
                                 n_commit, ws, ws_bytes);
  if (st) return st;
  UnmaskArgs args;
  fill_unmask(logits, n_rows, vocab, blk_off, n_blk, mode, n_div, threshold, masked, tokens, conf, n_commit, ws,
              &args);
  (void)hipGetLastError();
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_scan(logits, n_rows, vocab, masked, true, static_cast<ScanPartial*>(ws), s) != hipSuccess)
    return BC_ERR_HIP;
  return launch_unmask_decide(args, s) == hipSuccess ? BC_OK : BC_ERR_HIP;
}

size_t bc_verify_workspace_bytes(int32_t n_seq, int32_t n_lrows, int32_t vocab) {
  if (n_seq < 1 || n_lrows < 1 || vocab < 1 || (long long)n_seq * n_lrows > BC_MAX_SCAN_ROWS) return 0;
  return align256((size_t)n_seq * n_lrows * scan_chunks(vocab) * sizeof(ScanPartial));
}

int bc_spec_verify(const float* logits, int32_t n_seq, int32_t n_lrows, int32_t vocab, const int32_t* draft,
                   int32_t m, const uint8_t* fixed, const int32_t* first, int32_t* accept_len,
                   int32_t* bonus, void* ws, size_t ws_bytes, void* stream) {
  return spec_verify(logits, nullptr, 1.f, n_seq, n_lrows, vocab, draft, m, fixed, first, accept_len, bonus, ws,
                     ws_bytes, stream);
}

int bc_spec_verify_sampled(const float* logits, const float* noise, float inv_temperature, int32_t n_seq,
                           int32_t n_lrows, int32_t vocab, const int32_t* draft, int32_t m, const uint8_t* fixed,
                           const int32_t* first, int32_t* accept_len, int32_t* bonus, void* ws, size_t ws_bytes,
                           void* stream) {
  if (!noise) return BC_ERR_ARG;
  if (!std::isfinite(inv_temperature) || !(inv_temperature > 0.f)) return BC_ERR_ARG;
  return spec_verify(logits, noise, inv_temperature, n_seq, n_lrows, vocab, draft, m, fixed, first, accept_len,
                     bonus, ws, ws_bytes, stream);
}

}  // extern "C"
