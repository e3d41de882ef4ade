// Block-causal GQA attention over a committed KV prefix, split-KV flash-decode
// style, for gfx950.
//
// What is computed (WAM-Diff2 article sec. 2.1; Fast-dVLA notes, key design 1;
// Fast-dDrive method summary sec. 3.1 - 3.3): every active query row attends
// to all committed keys of its sequence (prefix, plus the rollout's private
// blocks under a shared-prefix fork) and to the active keys its block may see
// -- blocks are causal across, bidirectional (MDM pass) or causal (AR verify
// pass) inside.
//
// Work decomposition.  Query rows are grouped per KV head: row m of a group
// is (sequence, active row, query head within the GQA group), so one K/V
// stream serves all `group` query heads.  A workgroup (bf16: 4 waves x 16
// or 32 rows; fp32: 2 or 4 waves x 32 rows) takes one row tile against one
// key range and writes an unnormalised
// partial (reference max, sum, output) to its slot:
//   * prefix items: slot p < P covers chunk p of the committed prefix; under
//     a fork the tile runs over the rows of ALL rollouts, so the shared prefix
//     is streamed once per tile instead of once per rollout;
//   * active items: slot P covers the rollout's private keys plus the active
//     keys, where the block predicate applies (without a fork the active
//     keys may instead ride in the last prefix chunk's items: "fold", no
//     slot P).  The predicate is never stored:
//     active key j is visible to active row r iff j < lim(r), with lim(r) the
//     end of r's block (BIDIR) or r + 1 (CAUSAL).
// A second kernel merges the slots with log-sum-exp weights.
//
// MFMA mapping (bf16, v_mfma_f32_16x16x32_bf16).  Scores are computed
// transposed, S^T = K Q^T: K (16 keys x 32 dims) is the A operand read from
// LDS, Q^T is the B operand held in registers for the whole item.  The C
// layout gives each lane one query column and 4 key rows; with the key rows
// of the four 16-key tiles permuted so that tile pair (2s, 2s+1) gives lane
// group jj the keys 32s + 8jj .. 32s + 8jj + 7, the probabilities P^T are
// already laid out as the B operand of O^T = V^T P^T, so they never leave the
// registers.  The per-column softmax scalars (max, rescale) are per lane.
//
// Data movement (bf16).  K and V tiles of 64 keys go from HBM straight into
// LDS with buffer loads that write LDS (no staging registers), 1 KB per wave
// instruction, in two-stage rings of their own so that each load has a whole
// tile iteration to land; one barrier per tile.  Rows past a segment's end
// fall outside the buffer's record range and arrive as zeros.  Both tiles
// stay [key][dim] in LDS with a 16-byte-chunk XOR swizzle per row; K operands
// are plain 16-byte reads, V^T operands come from the transposing LDS read
// (ds_read_b64_tr_b16), which hands each lane 4 consecutive keys of one dim.
// Inside a wave the scores of tile j + 1 (MFMA) are computed while the
// probabilities of tile j (VALU) are formed.
// fp32 inputs (small configurations) use v_mfma_f32_16x16x4_f32 with
// register-staged tiles and the same softmax.

#include <type_traits>

#include "bc_internal.h"

#define BC_LDS __attribute__((address_space(3)))

namespace bc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t bf16_t;   // raw bf16 storage

constexpr float kNegInf = -__builtin_huge_valf();
// probabilities are allowed up to 2^kRescaleSlack before the reference max moves
constexpr float kRescaleSlack = 8.f;
// buffer descriptor word 3 for raw (untyped, stride 0) buffers on the gfx9 family
constexpr int kRawBufferWord3 = 0x00020000;

__device__ inline float wave_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// max over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the lane groups that
// hold one query column's keys).  v_permlane16_swap / v_permlane32_swap with
// both operands x return the two halves of each lane pair, so max of the
// pair is the max over l and l ^ 16 (l ^ 32); no LDS round trip.
__device__ inline float group4_max(float x) {
  const uint32_t b = __builtin_bit_cast(uint32_t, x);
  const auto p = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  x = fmaxf(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
  const uint32_t c = __builtin_bit_cast(uint32_t, x);
  const auto q = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)q[0]), __builtin_bit_cast(float, (uint32_t)q[1]));
}

// Workgroup barrier for LDS hand-offs only.  __syncthreads() also waits for
// every outstanding global load of the wave, which would stall on the next
// key tile's prefetch; here only LDS traffic is drained before the barrier.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Map
// hardware id -> logical id so that consecutive logical ids (the row tiles
// sharing one key chunk) land on the same XCD and share its L2.
__device__ inline int xcd_remap(int hw, int n) {
  const int per = n / 8, rem = n % 8;
  const int x = hw % 8, k = hw / 8;
  return x < rem ? x * (per + 1) + k : rem * (per + 1) + (x - rem) * per + k;
}

// Position inside the 64-key tile of the value held in C-register i of tile
// t: (lane-group offset) + (compile-time offset).  bf16: 32 (t >> 1) + 8 jj +
// 4 (t & 1) + i; fp32: 16 t + 4 jj + i.
template <bool kBf16> __device__ inline int key_group_off(int jj) { return kBf16 ? 8 * jj : 4 * jj; }
template <bool kBf16> constexpr int key_const_off(int t, int i) {
  return kBf16 ? 32 * (t >> 1) + 4 * (t & 1) + i : 16 * t + i;
}

// Row tile (group * n_mt_prefix + mt) that local tile jl of XCD x holds
// under the XCD-aligned mapping, or -1 past the last unit.
__device__ inline int xmap_tile(const AttnArgs& a, int x, int jl) {
  const int ju = fast_div(jl, a.dv_unit_tiles);
  const int unit = x + 8 * ju;
  if (unit >= a.n_units) return -1;
  return unit * a.unit_tiles + (jl - ju * a.unit_tiles);
}

// Logical item of this workgroup, or -1 for a workgroup with none.
// Key-chunk mapping (fork): workgroups are dispatched in block-id order, so
// the (long) prefix items take the lowest ids and start first; the short
// active items fill in behind them.  Within each class the XCD remap keeps
// neighbouring items -- the row tiles of one key chunk -- on one XCD.
// XCD-aligned mapping: workgroup 8 k + x is split k % n_slots of local row
// tile k / n_slots of XCD x (slot P: the active keys).
__device__ inline int item_of_block(const AttnArgs& a) {
  const int hw = blockIdx.x;
  if (a.xmap) {
    const int k = hw >> 3;
    const int jl = fast_div(k, a.dv_slots);
    const int slot = k - jl * a.n_slots;
    const int rt = xmap_tile(a, hw & 7, jl);
    if (rt < 0) return -1;
    const int grp = fast_div(rt, a.dv_mt_prefix);
    const int mt = rt - grp * a.n_mt_prefix;
    if (slot < a.n_splits) return (grp * a.n_splits + slot) * a.n_mt_prefix + mt;
    return a.n_prefix_items + grp * a.n_mt_active + mt;
  }
  if (hw < a.n_prefix_items) return xcd_remap(hw, a.n_prefix_items);
  return a.n_prefix_items + xcd_remap(hw - a.n_prefix_items, a.n_items - a.n_prefix_items);
}

// The kernel arguments are read with scalar loads that each CU's scalar
// cache meets cold.  Left to itself the compiler issues each load next to the
// field's first use, so the prologue waits for one round trip after another
// before the first K/V load can start.  These empty asm statements take the
// fields the item set-up needs as SGPR operands, so they are loaded in one
// burst at kernel start (measured: bs1 partial 6.15 -> 5.80 us).
__device__ inline void preload_item_args(const AttnArgs& a) {
  asm volatile("" ::"s"(a.n_prefix_items), "s"(a.n_items), "s"(a.n_mt_prefix), "s"(a.n_splits), "s"(a.fork),
               "s"(a.S), "s"(a.R), "s"(a.group), "s"(a.Hkv), "s"(a.Hq), "s"(a.n_mt_active), "s"(a.causal),
               "s"(a.n_blk));
  asm volatile("" ::"s"(a.dv_mt_prefix.mul), "s"(a.dv_mt_prefix.shift), "s"(a.dv_splits.mul),
               "s"(a.dv_splits.shift), "s"(a.dv_hkv.mul), "s"(a.dv_hkv.shift), "s"(a.dv_group.mul),
               "s"(a.dv_group.shift), "s"(a.chunk[0]), "s"(a.prefix_len[0]));
  asm volatile("" ::"s"(a.xmap), "s"(a.n_slots), "s"(a.unit_tiles), "s"(a.n_units), "s"(a.dv_slots.mul),
               "s"(a.dv_slots.shift), "s"(a.dv_unit_tiles.mul), "s"(a.dv_unit_tiles.shift));
}

// 16-byte chunk swizzles of the bf16 K and V tiles in LDS (row r of a tile,
// D / 8 chunks per row; chunk c of row r is stored at position c ^ swz(r)).
// swz_k spreads the 16 rows one K operand read touches (row bits 0, 1, 3, 4)
// over distinct chunk positions; swz_v does the same for the 4 rows x 32
// bytes per 16 lanes of a transposing V read (row bits 0, 1, 3).  Neither
// depends on row bits 2 and 5, so the per-tile row offsets of the reads stay
// immediates.
template <int D> __device__ inline int swz_k(int r) {
  if constexpr (D == 128) return (r & 3) | ((r >> 1) & 12);
  else return ((r >> 1) & 1) | ((r >> 2) & 6);
}
template <int D> __device__ inline int swz_v(int r) {
  if constexpr (D == 128) return ((r & 3) | ((r >> 1) & 4)) << 1;
  else return (((r >> 1) & 1) | ((r >> 2) & 2)) << 1;
}

// ---- what one workgroup computes: its row tile, slot and key segments
template <typename T>
struct Item {
  int g, mt, slot, s_item, rows_in_group;
  // the item's keys as at most two contiguous segments: the prefix chunk; or
  // the rollout's private keys, then the active keys (the only segment the
  // block predicate applies to)
  const T *k0, *v0, *k1, *v1;
  int n0, n1;
  bool masked0;
};

template <typename T, bool kDyn>
__device__ inline Item<T> decode_item(const AttnArgs& a, int item) {
  Item<T> it;
  it.k1 = it.v1 = nullptr;
  it.n1 = 0;
  it.masked0 = false;
  if (item < a.n_prefix_items) {
    const int rest = fast_div(item, a.dv_mt_prefix);
    it.mt = item - rest * a.n_mt_prefix;
    const int grp = fast_div(rest, a.dv_splits);
    it.slot = rest - grp * a.n_splits;
    int ps;
    if (a.fork) { it.g = grp; it.s_item = -1; ps = 0; it.rows_in_group = a.S * a.R * a.group; }
    else {
      it.s_item = fast_div(grp, a.dv_hkv);
      it.g = grp - it.s_item * a.Hkv;
      ps = it.s_item;
      it.rows_in_group = a.R * a.group;
    }
    const int key_begin = it.slot * a.chunk[ps];
    // (plan fields are the same for every lane; readfirstlane says so to the
    // compiler, which cannot tell through a generic pointer)
    const int plen = kDyn ? __builtin_amdgcn_readfirstlane(a.dyn->len) : a.prefix_len[ps];
    const int key_end = min(plen, key_begin + a.chunk[ps]);
    const long long off = ps * a.p_seq_stride + it.g * a.p_head_stride + (long long)key_begin * a.D;
    it.k0 = static_cast<const T*>(a.pk) + off;
    it.v0 = static_cast<const T*>(a.pv) + off;
    it.n0 = max(0, key_end - key_begin);
    if (a.fold && it.slot == a.n_splits - 1) {
      // the sequence's active keys ride in its last prefix chunk (no fork:
      // the item's rows are exactly the rows of that sequence and KV head)
      const long long act_off = (long long)(it.s_item * a.Hkv + it.g) * a.R * a.D;
      const T* ak = static_cast<const T*>(a.ak) + act_off;
      const T* av = static_cast<const T*>(a.av) + act_off;
      if (it.n0 > 0) {
        it.k1 = ak;
        it.v1 = av;
        it.n1 = a.R;
      } else {
        it.k0 = ak;
        it.v0 = av;
        it.n0 = a.R;
        it.masked0 = true;
      }
    }
  } else {
    const int i2 = item - a.n_prefix_items;
    const int rest = fast_div(i2, a.dv_mt_active);
    it.mt = i2 - rest * a.n_mt_active;
    it.s_item = fast_div(rest, a.dv_hkv);
    it.g = rest - it.s_item * a.Hkv;
    it.slot = a.n_splits;
    it.rows_in_group = a.R * a.group;
    const int lv = a.fork ? a.priv_len[it.s_item] : 0;
    const long long act_off = (long long)(it.s_item * a.Hkv + it.g) * a.R * a.D;
    const T* ak = static_cast<const T*>(a.ak) + act_off;
    const T* av = static_cast<const T*>(a.av) + act_off;
    if (lv > 0) {
      const long long prv_off = it.s_item * a.v_seq_stride + it.g * a.v_head_stride;
      it.k0 = static_cast<const T*>(a.vk) + prv_off;
      it.v0 = static_cast<const T*>(a.vv) + prv_off;
      it.n0 = lv;
      it.k1 = ak;
      it.v1 = av;
      it.n1 = a.R;
    } else {
      it.k0 = ak;
      it.v0 = av;
      it.n0 = a.R;
      it.masked0 = true;
    }
  }
  return it;
}

// this lane's two query columns: validity, output row, and the end of the
// active keys it may see
template <int CT, bool kDyn, typename T>
__device__ inline void lane_rows(const AttnArgs& a, const Item<T>& it, int row0, int n, bool (&valid)[CT],
                                 int (&orow)[CT], int (&lim)[CT]) {
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int m = row0 + c * 16 + n;
    valid[c] = m < it.rows_in_group;
    int s = it.s_item, rem = m;
    if (it.s_item < 0) { s = fast_div(m, a.dv_rows); rem = m - s * (a.R * a.group); }
    const int r = fast_div(rem, a.dv_group), hh = rem - r * a.group;
    orow[c] = valid[c] ? (s * a.R + r) * a.Hq + it.g * a.group + hh : 0;
    int l = r + 1;
    if (!a.causal) {
      l = a.R;
      if constexpr (kDyn) {
        const int nb = __builtin_amdgcn_readfirstlane(a.dyn->n_blk);
        for (int b = 0; b < nb; ++b) {
          const int e = __builtin_amdgcn_readfirstlane(a.dyn->blk_off[b + 1]);
          if (r < e) { l = e; break; }
        }
      } else {
        for (int b = 0; b < a.n_blk; ++b)
          if (r < a.blk_off[b + 1]) { l = a.blk_off[b + 1]; break; }
      }
    }
    lim[c] = l;
  }
}

// Online softmax over one 64-key tile held transposed in st (raw scores,
// one query column per lane and column tile); leaves the probabilities in st
// and rescales o when a column's reference max moves.  A tile inside an
// unmasked segment is fully visible: no predicate.  The scale is applied in
// the exponent, p = 2^(x * scale * log2 e - m) (scale > 0 keeps the order).
// Lazy rescale: the reference max only moves when the tile's max exceeds it
// by more than kRescaleSlack (log2 units), so after the first tiles the
// accumulator is almost never rescaled; probabilities stay below
// 2^kRescaleSlack and o, l and m stay consistent, so o / l is unchanged.
template <bool kBf16, int D, int CT>
__device__ inline void softmax_tile(f32x4 (&st)[CT][4], f32x4 (&o)[CT][D / 16], float (&m_run)[CT],
                                    float (&l_run)[CT], const int (&lim)[CT], int jj, int kb, int nkeys,
                                    bool masked, float sl2) {
  const bool full_tile = !masked && kb + kAttnKeyTile <= nkeys;
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    float tmax = kNegInf;
    if (!full_tile) {
      // visible iff key < nkeys (and key < lim for the active keys); with
      // key = kb + group offset + constant offset, one threshold per column
      const int thr = (masked ? min(nkeys, lim[c]) : nkeys) - kb - key_group_off<kBf16>(jj);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!(key_const_off<kBf16>(t, i) < thr)) st[c][t][i] = kNegInf;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, st[c][t][i]);
    tmax = group4_max(tmax);
    const float tm = tmax * sl2;
    const bool move = tm > m_run[c] + kRescaleSlack;
    const float mnew = move ? tm : m_run[c];
    const float muse = mnew == kNegInf ? 0.f : mnew;
    const float alpha = move ? __builtin_amdgcn_exp2f(m_run[c] - muse) : 1.f;
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[c][t][i], sl2, -muse));
        st[c][t][i] = p;
        psum += p;
      }
    l_run[c] = l_run[c] * alpha + psum;
    m_run[c] = mnew;
    if (__any(move)) {   // wave-uniform: skip when no column's reference moved
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[c][dt] *= alpha;
    }
  }
}

// this item's float32 partial for the lane's columns.  Non-temporal
// stores: the partials are read once, by the combine, so they are not kept
// in L2.  (kGroupSum: l_run holds each lane group's share of the column
// sum, added up here; otherwise every lane already holds the full sum)
template <int D, int CT, bool kGroupSum = true>
__device__ inline void write_partial_f32(const AttnArgs& a, int slot, const bool (&valid)[CT], const int (&orow)[CT],
                                         const float (&m_run)[CT], const float (&l_run)[CT],
                                         const f32x4 (&o)[CT][D / 16], int jj) {
  float* ws_o = static_cast<float*>(a.ws_o);
  float2* ws_ml = static_cast<float2*>(a.ws_ml);
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    float l = l_run[c];
    if constexpr (kGroupSum) {
      l += wave_xor(l, 16);
      l += wave_xor(l, 32);
    }
    if (!valid[c]) continue;
    const long long prow = (long long)slot * a.rows_total + orow[c];
    if (jj == 0) {
      __builtin_nontemporal_store(m_run[c], &ws_ml[prow].x);
      __builtin_nontemporal_store(l, &ws_ml[prow].y);
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      __builtin_nontemporal_store(o[c][dt], reinterpret_cast<f32x4*>(&ws_o[prow * D + 16 * dt + 4 * jj]));
  }
}

// this item's compact partial (bf16 inputs): the unnormalised output of a
// row is stored as int16 against one power of two per (slot, row),
//   h_d = round(32767 o_d 2^-e),  2^(e - 1) <= max_d |o_d| < 2^e,
// (v_cvt_pknorm_i16_f32: two values per instruction, rounded to nearest),
// so o_d = c h_d with c = 2^e / 32767, to within c / 2 <= 2^-15 max_d |o_d|.
// After the merge the error is at most 2^-15 of the largest |V| element
// the row attends to, far below the bf16 rounding of the output; the bytes
// per row and slot drop from 520 to 272.
// Every lane already holds its column's full sum in l_run.  A row's D
// values sit in the four lanes n, n + 16, n + 32, n + 48: lane group jj
// holds dims 16 dt + 4 jj + i.  Store k of a lane writes its values of
// dt = 2k and 2k + 1 (16 bytes) at record position 32 k + 8 jj, so the four
// lanes of a row fill 64 contiguous bytes per store instruction: position
// 32 k + 8 jj + 4 (dt & 1) + i holds dim 16 dt + 4 jj + i.
template <int D, int CT>
__device__ inline void write_partial_q16(const AttnArgs& a, int slot, const bool (&valid)[CT], const int (&orow)[CT],
                                         const float (&m_run)[CT], const float (&l_run)[CT],
                                         const f32x4 (&o)[CT][D / 16], int jj) {
  int16_t* ws_o = static_cast<int16_t*>(a.ws_o);
  f32x4* ws_ml = static_cast<f32x4*>(a.ws_ml);
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    float mo = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mo = fmaxf(mo, fabsf(o[c][dt][i]));
    mo = group4_max(mo);
    const int e = mo > 0.f ? __builtin_amdgcn_frexp_expf(mo) : 0;
    const float up = __builtin_amdgcn_ldexpf(1.f, -e);   // |o_d 2^-e| < 1
    if (!valid[c]) continue;
    const long long prow = (long long)slot * a.rows_total + orow[c];
    if (jj == 0)
      __builtin_nontemporal_store(f32x4{m_run[c], l_run[c], __builtin_amdgcn_ldexpf(1.f / 32767.f, e), 0.f},
                                  &ws_ml[prow]);
    u32x4 h[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const f32x4 x = o[c][dt] * up;
      const auto lo = __builtin_amdgcn_cvt_pknorm_i16(x[0], x[1]);
      const auto hi = __builtin_amdgcn_cvt_pknorm_i16(x[2], x[3]);
      h[dt >> 1][2 * (dt & 1)] = __builtin_bit_cast(uint32_t, lo);
      h[dt >> 1][2 * (dt & 1) + 1] = __builtin_bit_cast(uint32_t, hi);
    }
#pragma unroll
    for (int k = 0; k < D / 32; ++k)
      __builtin_nontemporal_store(h[k], reinterpret_cast<u32x4*>(&ws_o[prow * D + 32 * k + 8 * jj]));
  }
}

// ============================================================ bf16 partial
// One buffer-to-LDS load (the 16-byte form gfx950 adds): every lane fetches
// the 16 bytes at byte offset voff of the buffer described by rsrc and
// writes them to LDS at byte lds + 16 * lane; offsets at or past the
// buffer's size write zeros.  Inline assembly keeps the load out of the
// compiler's wait-count bookkeeping, which would otherwise make every LDS
// read wait for the loads filling the other stages; completion is awaited
// explicitly by tile_barrier().
// (M0 holds the LDS address; nothing else in these kernels uses M0, so the
// compiler's note that it reserves the register is silenced here.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void buffer_load_lds16(u32x4 rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc) : "memory", "m0");
}
#pragma clang diagnostic pop

// raw buffer descriptor: base, stride 0, num_records bytes
__device__ inline u32x4 raw_buffer(const void* base, int bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)b, (uint32_t)(b >> 32) & 0xffffu, (uint32_t)bytes, (uint32_t)kRawBufferWord3};
}

__device__ inline uint32_t lds_addr(const BC_LDS uint8_t* p) { return (uint32_t)reinterpret_cast<uintptr_t>(p); }

// LDS given at launch (the fork's row-tile form)
extern __shared__ __attribute__((aligned(16))) uint8_t bc_dyn_lds[];

__device__ inline uint32_t lds_offset(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((BC_LDS const uint8_t*)p);
}

// Barrier after this wave's buffer-to-LDS loads have landed and its LDS
// reads have returned: once every wave passes it, the stages loaded before
// it are visible to all waves and the stages read before it may be
// refilled.  (Encoding: vmcnt 0, lgkmcnt 0, expcnt unconstrained; as a
// builtin it also tells the compiler that every earlier load, e.g. of the Q
// operand, has completed.)
__device__ inline void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0070);
  asm volatile("s_barrier" ::: "memory");
}

// NW waves, each with CT column tiles of 16 query rows.
//
// Tile pipeline.  K and V sit in two-stage rings of their own: K(j) in
// k_st[j & 1], V(j) in v_st[j & 1].  Iteration j
//   1. starts the loads of K(j + 2) into K(j)'s stage and of V(j + 1) into
//      V(j - 1)'s stage (both were last read before the previous barrier);
//   2. takes tile j's maxima (its scores came from the previous iteration)
//      and, rarely, rescales the accumulator;
//   3. computes the scores of tile j + 1 (MFMA) while the probabilities of
//      tile j are formed (VALU): the two are independent, so the matrix and
//      vector units overlap inside one wave;
//   4. accumulates O^T += V(j)^T P(j)^T;
//   5. waits for its loads and meets the other waves at one barrier.
// Every load has a whole iteration to land.
template <int D, int NW, int CT, bool kDyn>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_partial_bf16_kernel(const AttnArgs a) {
  constexpr int KT = kAttnKeyTile;
  constexpr int RB = D * 2;            // bytes per key row
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int TB = KT * RB;          // bytes per tile and tensor
  constexpr int RPL = 1024 / RB;       // key rows per wave-wide 16-byte load
  static_assert(TB % (NW * 1024) == 0, "a tile must split evenly over the waves' 1 KB loads");
  constexpr int LPW = TB / (NW * 1024);  // loads per wave, tile and tensor
  constexpr int kWaveRows = 16 * CT;
  constexpr int kTileRows = NW * kWaveRows;
  __shared__ __attribute__((aligned(16))) uint8_t k_st0[TB], k_st1[TB], v_st0[TB], v_st1[TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, jj = lane >> 4;

  preload_item_args(a);
  if constexpr (kDyn) {   // device-resident plan: nothing to do once the decode has finished
    if (__builtin_amdgcn_readfirstlane(a.dyn->n) == 0) return;
  }
  const int item = item_of_block(a);
  if (item < 0) return;   // padding workgroup of the XCD-aligned mapping (uniform)
  const Item<bf16_t> it = decode_item<bf16_t, kDyn>(a, item);
  bool valid[CT];
  int orow[CT], lim[CT];
  lane_rows<CT, kDyn>(a, it, it.mt * kTileRows + wave * kWaveRows, n, valid, orow, lim);

  // ---- Q^T operand, resident for the whole item.  The two-column-tile
  // form loads it into registers here; the one-column-tile form stages it
  // through LDS in the prologue (below), so that the first score pass waits
  // for Q and K(0) only.
  const bf16_t* q = static_cast<const bf16_t*>(a.q);
  constexpr int QK = D / 32;
  bf16x8 qop[CT][QK];
  if constexpr (CT > 1) {
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int kk = 0; kk < QK; ++kk) {
        const bf16x8 z = {};
        qop[c][kk] = valid[c] ? *reinterpret_cast<const bf16x8*>(q + (long long)orow[c] * D + 32 * kk + 8 * jj) : z;
      }
  }

  // osum: the row sums, accumulated by the matrix core next to o (an
  // all-ones A operand), so that the normaliser sums exactly the bf16
  // probabilities the numerator uses; every lane holds its column's full sum
  float m_run[CT];
  f32x4 o[CT][D / 16], osum[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    m_run[c] = kNegInf;
    osum[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[c][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- load i of this wave fills stage bytes (wave LPW + i) 1024 + 16 lane,
  // i.e. key row (wave LPW + i) RPL + lane / CPR at chunk position
  // lane % CPR; it fetches the chunk the swizzle puts there (the swizzles
  // are XORs, so position and chunk map to each other the same way).  Also
  // the LDS addresses of the operand reads.
  uint32_t koff[LPW], voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int row = (wave * LPW + i) * RPL + lane / CPR, pos = lane % CPR;
    koff[i] = row * RB + (pos ^ swz_k<D>(row)) * 16;
    voff[i] = row * RB + (pos ^ swz_v<D>(row)) * 16;
  }
  uint32_t kaddr[QK], vaddr[D / 16];
  {
    const int kr = 8 * (n >> 2) + (n & 3);    // K row of tile 0 for A-operand row n
#pragma unroll
    for (int kk = 0; kk < QK; ++kk) kaddr[kk] = kr * RB + ((4 * kk + jj) ^ swz_k<D>(kr)) * 16;
    const int vr = 8 * jj + (n >> 2);         // V row read by this lane in a transposing read
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      vaddr[dt] = vr * RB + ((2 * dt + ((n & 3) >> 1)) ^ swz_v<D>(vr)) * 16 + (n & 1) * 8;
  }

  const int nt0 = (it.n0 + KT - 1) / KT;
  const int nt = nt0 + (it.n1 + KT - 1) / KT;

  // tile j of the item: its segment and first key
  auto tile_src = [&](int j, const bf16_t*& kp, const bf16_t*& vp, int& nk, int& kb, bool& msk)
                      __attribute__((always_inline)) {
    if (j < nt0) { kp = it.k0; vp = it.v0; nk = it.n0; kb = j * KT; msk = it.masked0; }
    else { kp = it.k1; vp = it.v1; nk = it.n1; kb = (j - nt0) * KT; msk = true; }
  };
  // loads of tile j's K or V into a stage; rows past the segment arrive as zeros
  auto load = [&](int j, bool is_v, const uint8_t* stage) __attribute__((always_inline)) {
    const bf16_t *kp, *vp;
    int nk, kb;
    bool msk;
    tile_src(j, kp, vp, nk, kb, msk);
    const u32x4 r = raw_buffer((is_v ? vp : kp) + (long long)kb * D, min(nk - kb, KT) * RB);
    const uint32_t dst = lds_offset(stage) + wave * LPW * 1024;
#pragma unroll
    for (int i = 0; i < LPW; ++i) buffer_load_lds16(r, dst + i * 1024, is_v ? voff[i] : koff[i]);
  };

  // S^T = K Q^T for 4 tiles of 16 keys x CT column tiles
  auto scores = [&](const uint8_t* stage, f32x4 (&st)[CT][4]) __attribute__((always_inline)) {
    const BC_LDS uint8_t* ks = (const BC_LDS uint8_t*)stage;
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t) st[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int trow = 32 * (t >> 1) + 4 * (t & 1);   // row offset of key tile t (swizzle-neutral bits)
      bf16x8 ka[QK];
#pragma unroll
      for (int kk = 0; kk < QK; ++kk) ka[kk] = *(const BC_LDS bf16x8*)(ks + kaddr[kk] + trow * RB);
#pragma unroll
      for (int kk = 0; kk < QK; ++kk)
#pragma unroll
        for (int c = 0; c < CT; ++c)
          st[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kk], qop[c][kk], st[c][t], 0, 0, 0);
    }
  };

  // keys of tile j a column may not see get -inf: past the segment's end,
  // and for the active keys past the column's limit
  auto mask = [&](int j, f32x4 (&st)[CT][4]) __attribute__((always_inline)) {
    const bf16_t *kp, *vp;
    int nk, kb;
    bool msk;
    tile_src(j, kp, vp, nk, kb, msk);
    if (msk || kb + KT > nk) {
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const int thr = (msk ? min(nk, lim[c]) : nk) - kb - key_group_off<true>(jj);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!(key_const_off<true>(t, i) < thr)) st[c][t][i] = kNegInf;
      }
    }
  };

  // Online softmax of one tile's scores (one query column per lane and
  // column tile), in two parts.  First the tile's maxima: the reference max
  // m only moves when a column's tile max exceeds it by more than
  // kRescaleSlack, so after the first tiles the accumulator is almost never
  // rescaled; returns whether any column of the wave moved, with the
  // columns' rescale factors and the max the exponents use.
  auto maxima = [&](const f32x4 (&st)[CT][4], float (&alpha)[CT], float (&muse)[CT]) __attribute__((always_inline)) {
    const float sl2 = a.scale_log2;
    bool moved = false;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      float tmax = kNegInf;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, st[c][t][i]);
      tmax = group4_max(tmax);
      const float tm = tmax * sl2;
      const bool move = tm > m_run[c] + kRescaleSlack;
      const float mnew = move ? tm : m_run[c];
      muse[c] = mnew == kNegInf ? 0.f : mnew;
      alpha[c] = move ? __builtin_amdgcn_exp2f(m_run[c] - muse[c]) : 1.f;
      m_run[c] = mnew;
      moved |= move;
    }
    return moved;
  };
  // Then the probabilities p = 2^(x scale log2 e - m), their row sums and
  // their bf16 B operands for the PV product.
  auto probs = [&](const f32x4 (&st)[CT][4], const float (&alpha)[CT], const float (&muse)[CT],
                   bf16x8 (&pb)[CT][2]) __attribute__((always_inline)) {
    const float sl2 = a.scale_log2;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      float p[4][4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[t][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[c][t][i], sl2, -muse[c]));
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pb[c][s2][e] = (__bf16)p[2 * s2][e];
          pb[c][s2][e + 4] = (__bf16)p[2 * s2 + 1][e];
        }
    }
  };

  // O^T += V^T P^T
  auto accumulate = [&](const uint8_t* stage, const bf16x8 (&pb)[CT][2]) __attribute__((always_inline)) {
    const BC_LDS uint8_t* vs = (const BC_LDS uint8_t*)stage;
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int c = 0; c < CT; ++c) osum[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[c][s2], osum[c], 0, 0, 0);
#pragma unroll
    for (int dt0 = 0; dt0 < D / 16; dt0 += 4) {
      bf16x8 va[4][2];
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          // keys 32 s2 + 8 jj + 0..3 and + 4..7 of dim 16 (dt0 + d4) + n
          const BC_LDS uint8_t* base = vs + vaddr[dt0 + d4] + 32 * s2 * RB;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BC_LDS i16x4*)base);
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BC_LDS i16x4*)(base + 4 * RB));
          va[d4][s2] = __builtin_bit_cast(bf16x8, (i16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int c = 0; c < CT; ++c)
            o[c][dt0 + d4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[d4][s2], pb[c][s2], o[c][dt0 + d4], 0, 0, 0);
    }
  };

  // iteration j (parity fixed per unrolled half): s_cur holds the scores of
  // tile j, s_nxt receives those of tile j + 1.  The last form has no next
  // tile: no score pass and no closing barrier.
  auto step = [&](auto par, auto last, int j, f32x4 (&s_cur)[CT][4], f32x4 (&s_nxt)[CT][4])
                  __attribute__((always_inline)) {
    constexpr bool odd = decltype(par)::value;
    constexpr bool kLast = decltype(last)::value;
    if constexpr (!kLast) {
      if (j + 2 < nt) load(j + 2, false, odd ? k_st1 : k_st0);
      if (j + 1 < nt) load(j + 1, true, odd ? v_st0 : v_st1);
    }
    mask(j, s_cur);
    float alpha[CT], muse[CT];
    if (__any(maxima(s_cur, alpha, muse))) {   // wave-uniform
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[c][dt] *= alpha[c];
#pragma unroll
      for (int c = 0; c < CT; ++c) osum[c] *= alpha[c];
    }
    // one branch-free block: the scheduler interleaves the score MFMAs of
    // tile j + 1 with the exponentials of tile j, then the PV MFMAs.  With
    // two column tiles it runs at raised wave priority, so that of the two
    // waves sharing a SIMD the one issuing MFMAs is preferred and the
    // other's vector work fills the gaps.
    if constexpr (CT > 1) __builtin_amdgcn_s_setprio(1);
    if constexpr (!kLast) scores(odd ? k_st0 : k_st1, s_nxt);
    bf16x8 pb[CT][2];
    probs(s_cur, alpha, muse, pb);
    accumulate(odd ? v_st1 : v_st0, pb);
    if constexpr (CT > 1) {
      // Left alone, the scheduler issues the score MFMAs back to back and
      // the exponentials after them, and each operand read right before
      // its MFMA, so every MFMA pair waits out an LDS round trip.  Instead:
      // each score MFMA is followed by three vector instructions (an MFMA
      // occupies the matrix core for 16 cycles and the issue port for
      // about 6; an exponential costs about three FMAs); the K operand
      // reads run one 16-key step ahead of their MFMAs; the PV MFMAs start
      // with the four row-sum MFMAs (no LDS operand) behind the first V
      // reads, and each later pair of V reads is issued two MFMA pairs
      // ahead of its use.  (Measured at N = 64 rollouts: partial 55.5 ->
      // 53.4 us; reads four steps ahead, or V reads further ahead, were no
      // better.)
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);       // K reads, steps 0 and 1
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // VALU
        }
        if (t < 2) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // K reads, step t + 2
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);       // the first two V read pairs
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);       // row-sum MFMAs
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);     // PV MFMA pair
        if (u < 14) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // the V read pair two ahead
      }
      __builtin_amdgcn_s_setprio(0);
    }
    if constexpr (!kLast) tile_barrier();
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using More = std::false_type;
  using Last = std::true_type;
  // One-column-tile form: the Q tile (kTileRows rows of RB bytes, the size
  // of one stage) goes into V(1)'s stage, which iteration 0 refills only
  // after the barrier that follows the first score pass.  Each wave loads
  // its own 16 rows; the row a load lane needs is the output row that
  // lane_rows gave lane (its row within the wave), fetched with a shuffle.
  // Tile row t lands at t RB with 16-byte chunk c at position c ^ (t mod
  // CPR), so the 16 lanes reading one chunk of 16 consecutive rows hit
  // distinct banks.  Rows past the item's rows load the wave's first row
  // (real data in unused columns); a wave without rows loads zeros.
  auto load_q = [&](const uint8_t* stage) __attribute__((always_inline)) {
    const int mine = valid[0] ? orow[0] : -1;
    const int base = __builtin_amdgcn_readfirstlane(mine);
    const u32x4 rsrc = raw_buffer(q + (long long)max(base, 0) * D, base >= 0 ? 0x7ffffff0 : 0);
    const uint32_t dst = lds_offset(stage) + wave * LPW * 1024;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int src = i * RPL + lane / CPR, pos = lane % CPR;   // row within the wave
      const int ro = __shfl(mine, src, 64);
      const uint32_t off = (uint32_t)((ro >= 0 ? ro - base : 0) * RB + (pos ^ (src % CPR)) * 16);
      buffer_load_lds16(rsrc, dst + i * 1024, off);
    }
  };

  f32x4 sa[CT][4], sb[CT][4];
  if (nt > 0) {
    // K(0) first: its loads need only the item, while the Q tile's wait for
    // the row shuffles (measured: bs1 partial 5.83 -> 5.76 us)
    load(0, false, k_st0);
    if constexpr (CT == 1) load_q(v_st1);
    load(0, true, v_st0);
    if (nt > 1) load(1, false, k_st1);
  }
  if constexpr (CT == 1) {
    // K(0) and Q have landed once no more than the loads issued after them
    // (V(0), and K(1) when there is a second tile) are outstanding
    if (nt > 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPW) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPW) : "memory");
    asm volatile("s_barrier" ::: "memory");
    const BC_LDS uint8_t* qs = (const BC_LDS uint8_t*)v_st1;
    const int t = wave * kWaveRows + n;
#pragma unroll
    for (int kk = 0; kk < QK; ++kk)
      qop[0][kk] = *(const BC_LDS bf16x8*)(qs + t * RB + ((4 * kk + jj) ^ (t % CPR)) * 16);
  } else {
    tile_barrier();
  }
  if (nt > 0) scores(k_st0, sa);
  // every wave has read K(0) (and, one-column-tile form, the Q tile) before
  // iteration 0 refills those stages; V(0) and K(1) have landed
  if (CT == 1 ? nt > 0 : nt > 2) tile_barrier();
  if constexpr (CT == 1) {
    // few rows, short items: the last iteration gets its own form
    int j = 0;
    for (; j + 2 < nt; j += 2) {
      step(S0{}, More{}, j, sa, sb);
      step(S1{}, More{}, j + 1, sb, sa);
    }
    if (j + 1 < nt) {
      step(S0{}, More{}, j, sa, sb);
      step(S1{}, Last{}, j + 1, sb, sa);
    } else if (j < nt) {
      step(S0{}, Last{}, j, sa, sb);
    }
  } else {
    // long items: one form only (a second would push the register
    // allocation past the budget); the last score pass reads a stale stage
    // and is discarded
    for (int j = 0; j < nt; j += 2) {
      step(S0{}, More{}, j, sa, sb);
      if (j + 1 < nt) step(S1{}, More{}, j + 1, sb, sa);
    }
  }

  float l_run[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) l_run[c] = osum[c][0];
  if (a.compact) write_partial_q16<D, CT>(a, it.slot, valid, orow, m_run, l_run, o, jj);
  else write_partial_f32<D, CT, false>(a, it.slot, valid, orow, m_run, l_run, o, jj);
}

// ==================================================== fork, row-tile form
// Shared-prefix fork with every CU the same work: row tile (kv head g,
// rollout s, half h) holds half of rollout s's R x group query rows of kv
// head g (at most 96), and P key splits of it make the workgroups (2 N Hkv
// P >= the CUs; P = 1 at N = 64, 4 at N = 16).  Split q covers the shared
// prefix's chunk [q C, (q + 1) C); the last split also the rollout's private
// keys and the active keys.  The workgroup covers its split's keys in two
// halves:
//   kh = 0: the first part of the chunk, then (last split) the private keys;
//   kh = 1: the rest of the chunk, then (last split) the active keys (the
//           only segment the block predicate applies to),
// cut so that both halves run the same number of 64-key tiles (the shorter
// runs one empty tile at most).  Wave 6 kh + rg holds row group rg (16 rows,
// one column tile) of key half kh: 12 waves, three per SIMD, which hide each
// other's latencies.  Each half streams its keys through a two-stage K/V ring
// of its own, loaded by its first two waves.  At the end half 1 hands (o,
// m, l) to half 0 through LDS, which merges them and writes, with one split,
// the normalised output (no split partials, no combine) and otherwise the
// split's record for the combine.  The price is one K and one V operand read
// per 16 rows instead of per 32 (two column tiles per wave leave 6 waves,
// which sit unevenly on the 4 SIMDs: measured slower, 67.7 against 61.5 us).
// LDS (given at launch): per half K(0), K(1), V(0), V(1) (64 KB), then the
// Q tile of the 96 rows (24 KB).
constexpr int kForkRG = kForkTileRows / 16;   // 6 row groups per key half
constexpr unsigned kForkLdsBytes = 2u * 4 * kAttnKeyTile * 128 * 2 + kForkTileRows * 128 * 2;

template <int D>
__global__ __launch_bounds__(2 * kForkRG * 64) __attribute__((amdgpu_waves_per_eu(3)))
void attn_fork_rows_kernel(const AttnArgs a) {
  constexpr int RG = kForkRG;
  constexpr int CT = 1;                // one 16-row column tile per wave
  constexpr int KT = kAttnKeyTile;
  constexpr int RB = D * 2;            // bytes per key row
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int TB = KT * RB;          // bytes per tile and tensor
  constexpr int RPL = 1024 / RB;       // key rows per wave-wide 16-byte load
  constexpr int WR = 16;               // rows per wave
  // loading waves per half: two, one per SIMD across both halves (measured
  // at N = 64, draft / verify pass: four 59.5 / 57.3 us, two 57.0 / 54.4 us,
  // one 64.1 / 60.0 us)
  constexpr int LW = 2;
  static_assert(TB % (LW * 1024) == 0 && LW <= RG, "a tile must split evenly over the loading waves");
  constexpr int LPW = TB / (LW * 1024);
  constexpr int QLPW = WR * RB / 1024;  // Q loads per wave (its rows)
  constexpr int QK = D / 32;
  constexpr int kHalfBytes = 4 * TB;
  constexpr uint32_t kQOff = 2 * kHalfBytes;
  using lds_t = const BC_LDS uint8_t*;
  const lds_t lds = (lds_t)bc_dyn_lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = w / RG, rg = w - kh * RG;
  const int n = lane & 15, jj = lane >> 4;

  // workgroup: (kv head g, key split q, rollout s, half hf), in that order
  // of significance, so that consecutive ones -- the row tiles streaming one
  // prefix chunk -- share an XCD and its L2.  (Integer division runs on the
  // vector unit; readfirstlane keeps these workgroup-uniform values, and the
  // pointers made from them, in SGPRs.)
  const int per_g = a.n_splits * a.S * 2;
  const int id = __builtin_amdgcn_readfirstlane(xcd_remap(blockIdx.x, a.Hkv * per_g));
  const int g = __builtin_amdgcn_readfirstlane(id / per_g);
  const int q = __builtin_amdgcn_readfirstlane((id - g * per_g) / (a.S * 2));
  const int tile = id - g * per_g - q * a.S * 2;
  const int s = tile >> 1, hf = tile & 1;
  const int rows_r = a.R * a.group;
  const int half = (rows_r + 1) >> 1;
  const int rows_here = hf == 0 ? half : rows_r - half;
  // output row of row ml of the tile (clamped to the tile's last row)
  auto out_row = [&](int ml, int& r) __attribute__((always_inline)) {
    const int mr = hf * half + min(ml, rows_here - 1);
    r = mr / a.group;
    return (s * a.R + r) * a.Hq + g * a.group + (mr - r * a.group);
  };

  // this lane's query columns
  bool valid[CT];
  int orow[CT], lim[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int ml = rg * WR + c * 16 + n;
    valid[c] = ml < rows_here;
    int r;
    orow[c] = out_row(ml, r);
    int l = r + 1;
    if (!a.causal) {
      l = a.R;
      for (int b = 0; b < a.n_blk; ++b)
        if (r < a.blk_off[b + 1]) { l = a.blk_off[b + 1]; break; }
    }
    lim[c] = l;
  }

  // split q's keys: the prefix chunk [q C, min(L, (q + 1) C)), and in the
  // last split also the rollout's private keys and the active keys; the two
  // halves' segments, both run nt tiles
  const int L = a.prefix_len[0], C = a.chunk[0];
  const int k0 = min(L, q * C);
  const int nc = min(L, k0 + C) - k0;
  const bool last = q == a.n_splits - 1;
  const int lv = last ? a.priv_len[s] : 0, ra = last ? a.R : 0;
  const int TL = (nc + KT - 1) / KT, tv = (lv + KT - 1) / KT, tr = (ra + KT - 1) / KT;
  const int cut = __builtin_amdgcn_readfirstlane(max(0, min(TL, (TL + tr - tv) / 2)));
  const int X = min(cut * KT, nc);
  const int nt = __builtin_amdgcn_readfirstlane(max(cut + tv, TL - cut + tr));
  const bf16_t* pk = static_cast<const bf16_t*>(a.pk) + g * a.p_head_stride + (long long)k0 * D;
  const bf16_t* pv = static_cast<const bf16_t*>(a.pv) + g * a.p_head_stride + (long long)k0 * D;
  const bf16_t *ka, *va, *kb_, *vb_;
  int na, nb;
  if (kh == 0) {
    ka = pk;
    va = pv;
    na = X;
    const long long po = s * a.v_seq_stride + g * a.v_head_stride;
    kb_ = static_cast<const bf16_t*>(a.vk) + po;
    vb_ = static_cast<const bf16_t*>(a.vv) + po;
    nb = lv;
  } else {
    ka = pk + (long long)X * D;
    va = pv + (long long)X * D;
    na = nc - X;
    const long long ao = (long long)(s * a.Hkv + g) * a.R * D;
    kb_ = static_cast<const bf16_t*>(a.ak) + ao;
    vb_ = static_cast<const bf16_t*>(a.av) + ao;
    nb = ra;
  }
  const int nta = (na + KT - 1) / KT, ntb = (nb + KT - 1) / KT;
  const bool mskb = kh == 1;

  // tile j of this half: its segment, first key, key count and whether the
  // block predicate applies; past both segments an empty tile (no keys)
  auto tile_src = [&](int j, const bf16_t*& kp, const bf16_t*& vp, int& nk, int& kb, bool& msk)
                      __attribute__((always_inline)) {
    if (j < nta) { kp = ka; vp = va; nk = na; kb = j * KT; msk = false; }
    else if (j < nta + ntb) { kp = kb_; vp = vb_; nk = nb; kb = (j - nta) * KT; msk = mskb; }
    else { kp = ka; vp = va; nk = 0; kb = 0; msk = false; }
  };

  // LDS addresses: this half's stages at hb; operand addresses include hb
  const uint32_t hb = kh * kHalfBytes;
  uint32_t koff[LPW], voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int row = (rg * LPW + i) * RPL + lane / CPR, pos = lane % CPR;
    koff[i] = row * RB + (pos ^ swz_k<D>(row)) * 16;
    voff[i] = row * RB + (pos ^ swz_v<D>(row)) * 16;
  }
  uint32_t kaddr[QK], vaddr[D / 16];
  {
    const int kr = 8 * (n >> 2) + (n & 3);
#pragma unroll
    for (int kk = 0; kk < QK; ++kk) kaddr[kk] = hb + kr * RB + ((4 * kk + jj) ^ swz_k<D>(kr)) * 16;
    const int vr = 8 * jj + (n >> 2);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      vaddr[dt] = hb + vr * RB + ((2 * dt + ((n & 3) >> 1)) ^ swz_v<D>(vr)) * 16 + (n & 1) * 8;
  }
  // loads of tile j's K or V into stage p of this half (K at p TB, V at
  // (2 + p) TB), by the half's first LW waves; rows past the tile's keys
  // arrive as zeros
  auto load = [&](int j, bool is_v, int p) __attribute__((always_inline)) {
    if (rg >= LW) return;   // wave-uniform
    const bf16_t *kp, *vp;
    int nk, kb;
    bool msk;
    tile_src(j, kp, vp, nk, kb, msk);
    // (the clamp compiles to a vector med3: readfirstlane keeps the
    // descriptor in SGPRs, as the buffer load needs)
    const int nrec = __builtin_amdgcn_readfirstlane(max(0, min(nk - kb, KT)) * RB);
    const u32x4 rs = raw_buffer((is_v ? vp : kp) + (long long)kb * D, nrec);
    const uint32_t dst = lds_addr(lds) + hb + (is_v ? 2 + p : p) * TB + rg * LPW * 1024;
#pragma unroll
    for (int i = 0; i < LPW; ++i) buffer_load_lds16(rs, dst + i * 1024, is_v ? voff[i] : koff[i]);
  };

  bf16x8 qop[CT][QK];
  float m_run[CT];
  f32x4 o[CT][D / 16], osum[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    m_run[c] = kNegInf;
    osum[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[c][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto scores = [&](int p, f32x4 (&st)[CT][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t) st[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int trow = 32 * (t >> 1) + 4 * (t & 1);
      bf16x8 kop[QK];
#pragma unroll
      for (int kk = 0; kk < QK; ++kk) kop[kk] = *(const BC_LDS bf16x8*)(lds + kaddr[kk] + p * TB + trow * RB);
#pragma unroll
      for (int kk = 0; kk < QK; ++kk)
#pragma unroll
        for (int c = 0; c < CT; ++c)
          st[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kk], qop[c][kk], st[c][t], 0, 0, 0);
    }
  };
  auto mask = [&](int j, f32x4 (&st)[CT][4]) __attribute__((always_inline)) {
    const bf16_t *kp, *vp;
    int nk, kb;
    bool msk;
    tile_src(j, kp, vp, nk, kb, msk);
    if (msk || kb + KT > nk) {
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const int thr = (msk ? min(nk, lim[c]) : nk) - kb - key_group_off<true>(jj);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!(key_const_off<true>(t, i) < thr)) st[c][t][i] = kNegInf;
      }
    }
  };
  auto accumulate = [&](int p, const bf16x8 (&pb)[CT][2]) __attribute__((always_inline)) {
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int c = 0; c < CT; ++c) osum[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[c][s2], osum[c], 0, 0, 0);
#pragma unroll
    for (int dt0 = 0; dt0 < D / 16; dt0 += 4) {
      bf16x8 vop[4][2];
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const lds_t base = lds + vaddr[dt0 + d4] + (2 + p) * TB + 32 * s2 * RB;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BC_LDS i16x4*)base);
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BC_LDS i16x4*)(base + 4 * RB));
          vop[d4][s2] = __builtin_bit_cast(bf16x8, (i16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int c = 0; c < CT; ++c)
            o[c][dt0 + d4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[d4][s2], pb[c][s2], o[c][dt0 + d4], 0, 0, 0);
    }
  };
  // iteration j: as the partial kernel's (maxima and rare rescale of tile j,
  // score MFMAs of tile j + 1 beside the exponentials of tile j, PV MFMAs
  // of tile j, one barrier).  The MFMA block runs at raised wave priority,
  // so that of the three waves sharing a SIMD the one issuing MFMAs is
  // preferred (measured: 61.5 -> 59.5 us per N = 64 draft pass).
  auto step = [&](auto par, auto last, int j, f32x4 (&s_cur)[CT][4], f32x4 (&s_nxt)[CT][4])
                  __attribute__((always_inline)) {
    constexpr int p = decltype(par)::value;
    constexpr bool kLast = decltype(last)::value;
    mask(j, s_cur);
    const float sl2 = a.scale_log2;
    float alpha[CT], muse[CT];
    bool moved = false;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      float tmax = kNegInf;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, s_cur[c][t][i]);
      tmax = group4_max(tmax);
      const float tm = tmax * sl2;
      const bool move = tm > m_run[c] + kRescaleSlack;
      const float mnew = move ? tm : m_run[c];
      muse[c] = mnew == kNegInf ? 0.f : mnew;
      alpha[c] = move ? __builtin_amdgcn_exp2f(m_run[c] - muse[c]) : 1.f;
      m_run[c] = mnew;
      moved |= move;
    }
    if (__any(moved)) {
#pragma unroll
      for (int c = 0; c < CT; ++c) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[c][dt] *= alpha[c];
        osum[c] *= alpha[c];
      }
    }
    __builtin_amdgcn_s_setprio(1);
    if constexpr (!kLast) scores(1 - p, s_nxt);
    // the loading waves issue the next tiles' loads after their score MFMAs,
    // not before: the MFMAs start sooner and the loads still have most of an
    // iteration to land (measured at N = 64, draft / verify: 57.6 / 55.6 ->
    // 56.2 / 54.5 us; in the split-plan kernel the same move cost the
    // batch-16 call 3 us cold, whose loads need the whole iteration)
    if constexpr (!kLast) {
      if (j + 2 < nt) load(j + 2, false, p);
      if (j + 1 < nt) load(j + 1, true, 1 - p);
    }
    bf16x8 pb[CT][2];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      float pr[4][4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[t][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[c][t][i], sl2, -muse[c]));
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pb[c][s2][e] = (__bf16)pr[2 * s2][e];
          pb[c][s2][e + 4] = (__bf16)pr[2 * s2 + 1][e];
        }
    }
    accumulate(p, pb);
    __builtin_amdgcn_s_setprio(0);
    if constexpr (!kLast) tile_barrier();
  };

  // ---- prologue: K(0), (half 0) the Q tile, V(0), K(1)
  load(0, false, 0);
  if (kh == 0) {
    // this wave's WR Q rows, row t of the wave at t RB with chunk c at
    // position c ^ (t mod CPR); rows past the tile's rows load its last row
    const bf16_t* q = static_cast<const bf16_t*>(a.q);
    int r0;
    const int base = __builtin_amdgcn_readfirstlane(out_row(rg * WR, r0));
    const u32x4 rs = raw_buffer(q + (long long)base * D, 0x7ffffff0);
    const uint32_t dst = lds_addr(lds) + kQOff + rg * WR * RB;
#pragma unroll
    for (int i = 0; i < QLPW; ++i) {
      const int t = i * RPL + lane / CPR, pos = lane % CPR;   // row within the wave
      int rt;
      const int ro = out_row(rg * WR + t, rt);
      buffer_load_lds16(rs, dst + i * 1024, (uint32_t)((ro - base) * RB + (pos ^ (t % CPR)) * 16));
    }
  }
  load(0, true, 0);
  if (nt > 1) load(1, false, 1);
  // K(0) and Q have landed once no more than V(0) and K(1) are outstanding
  if (rg < LW) {
    if (nt > 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPW) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPW) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  asm volatile("s_barrier" ::: "memory");
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int t = rg * WR + c * 16 + n;
#pragma unroll
    for (int kk = 0; kk < QK; ++kk)
      qop[c][kk] = *(const BC_LDS bf16x8*)(lds + kQOff + t * RB + ((4 * kk + jj) ^ (t % CPR)) * 16);
  }
  f32x4 sa[CT][4], sb[CT][4];
  scores(0, sa);
  tile_barrier();

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using More = std::false_type;
  using Last = std::true_type;
  int j = 0;
  for (; j + 2 < nt; j += 2) {
    step(S0{}, More{}, j, sa, sb);
    step(S1{}, More{}, j + 1, sb, sa);
  }
  if (j + 1 < nt) {
    step(S0{}, More{}, j, sa, sb);
    step(S1{}, Last{}, j + 1, sb, sa);
  } else {
    step(S0{}, Last{}, j, sa, sb);
  }

  // ---- half 1 hands (o, m, l) to half 0 through its own (now idle) stages
  constexpr int kPub = CT * ((D / 16) * 1024 + 2 * 256);
  static_assert(RG * kPub <= kHalfBytes, "published partials fit in half 1's stages");
  float l_run[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) l_run[c] = osum[c][0];
  lds_barrier();
  BC_LDS uint8_t* const pub = (BC_LDS uint8_t*)(lds + kHalfBytes + rg * kPub);
  if (kh == 1) {
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      BC_LDS uint8_t* pc = pub + c * ((D / 16) * 1024 + 512);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) *(BC_LDS f32x4*)(pc + dt * 1024 + lane * 16) = o[c][dt];
      *(BC_LDS float*)(pc + (D / 16) * 1024 + lane * 4) = m_run[c];
      *(BC_LDS float*)(pc + (D / 16) * 1024 + 256 + lane * 4) = l_run[c];
    }
  }
  lds_barrier();
  if (kh == 1) return;
  // merge half 1's (o, m, l) into half 0's
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const BC_LDS uint8_t* pc = pub + c * ((D / 16) * 1024 + 512);
    const float m1 = *(const BC_LDS float*)(pc + (D / 16) * 1024 + lane * 4);
    const float l1 = *(const BC_LDS float*)(pc + (D / 16) * 1024 + 256 + lane * 4);
    const float m = fmaxf(m_run[c], m1);
    if (m != kNegInf) {
      const float a0 = __builtin_amdgcn_exp2f(m_run[c] - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[c][dt] = o[c][dt] * a0 + *(const BC_LDS f32x4*)(pc + dt * 1024 + lane * 16) * a1;
      l_run[c] = l_run[c] * a0 + l1 * a1;
      m_run[c] = m;
    }
  }
  if (!a.direct) {
    // one of several key splits: the split record for the combine
    if (a.compact) write_partial_q16<D, CT>(a, q, valid, orow, m_run, l_run, o, jj);
    else write_partial_f32<D, CT, false>(a, q, valid, orow, m_run, l_run, o, jj);
    return;
  }
  // the only split: the normalised output
  bf16_t* out = static_cast<bf16_t*>(a.out);
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    if (!valid[c]) continue;
    const float inv = l_run[c] > 0.f ? 1.f / l_run[c] : 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const f32x4 x = o[c][dt] * inv;
      uint16_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = __builtin_bit_cast(uint16_t, (__bf16)x[e]);
      *reinterpret_cast<u32x2*>(out + (long long)orow[c] * D + 16 * dt + 4 * jj) =
          u32x2{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16)};
    }
  }
}

// ============================================================ fp32 partial
// Register-staged: the next tile's global loads are issued before the
// current tile is computed and written to LDS one iteration later.  Loads
// past a segment's end are clamped to its last key: finite data that the
// softmax gives probability 0.
template <int D, int NW, bool kDyn>
__global__ __launch_bounds__(NW * 64) void attn_partial_f32_kernel(const AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int KT = kAttnKeyTile;
  constexpr int KP = D + 4;                    // LDS row pitch (elements)
  constexpr int kWaveRows = 32;                // 2 column tiles of 16 rows
  constexpr int kTileRows = NW * kWaveRows;
  __shared__ __attribute__((aligned(16))) float k_lds[KT * KP];
  __shared__ __attribute__((aligned(16))) float v_lds[KT * KP];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, jj = lane >> 4;

  if constexpr (kDyn) {   // device-resident plan: nothing to do once the decode has finished
    if (__builtin_amdgcn_readfirstlane(a.dyn->n) == 0) return;
  }
  const int item = item_of_block(a);
  if (item < 0) return;   // padding workgroup of the XCD-aligned mapping (uniform)
  const Item<float> it = decode_item<float, kDyn>(a, item);
  bool valid[2];
  int orow[2], lim[2];
  lane_rows<2, kDyn>(a, it, it.mt * kTileRows + wave * kWaveRows, n, valid, orow, lim);

  const float* q = static_cast<const float*>(a.q);
  constexpr int QK = D / 4;
  float qop[2][QK];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int kk = 0; kk < QK; ++kk) qop[c][kk] = valid[c] ? q[(long long)orow[c] * D + 4 * kk + jj] : 0.f;

  float m_run[2] = {kNegInf, kNegInf};
  float l_run[2] = {0.f, 0.f};
  f32x4 o[2][D / 16];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[c][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int CPR = D / 4;                   // 16-byte units per key row
  constexpr int NK = (KT * CPR + NT - 1) / NT; // units per thread
  u32x4 kreg[NK], vreg[NK];
  auto load_tile = [&](const float* kp, const float* vp, int nkeys, int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const int idx = tid + NT * u;
      const int kr = min(idx / CPR, KT - 1), cc = idx % CPR;
      const long long off = (long long)min(kb + kr, nkeys - 1) * D + 4 * cc;
      kreg[u] = *reinterpret_cast<const u32x4*>(kp + off);
      vreg[u] = *reinterpret_cast<const u32x4*>(vp + off);
    }
  };
  auto store_tile = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const int idx = tid + NT * u;
      if (idx >= KT * CPR) continue;
      const int kr = idx / CPR, cc = idx % CPR;
      *reinterpret_cast<u32x4*>(&k_lds[kr * KP + 4 * cc]) = kreg[u];
      *reinterpret_cast<u32x4*>(&v_lds[kr * KP + 4 * cc]) = vreg[u];
    }
  };

  const float sl2 = a.scale_log2;
  auto process_tile = [&](int kb, int nkeys, bool masked) __attribute__((always_inline)) {
    f32x4 st[2][4];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t) st[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int kk = 0; kk < QK; ++kk) {
        const float ka = k_lds[(16 * t + n) * KP + 4 * kk + jj];
#pragma unroll
        for (int c = 0; c < 2; ++c)
          st[c][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka, qop[c][kk], st[c][t], 0, 0, 0);
      }
    softmax_tile<false, D, 2>(st, o, m_run, l_run, lim, jj, kb, nkeys, masked, sl2);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float va = v_lds[(16 * t + 4 * jj + i) * KP + 16 * dt + n];
#pragma unroll
          for (int c = 0; c < 2; ++c)
            o[c][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va, st[c][t][i], o[c][dt], 0, 0, 0);
        }
  };

  for (int sgi = 0; sgi < 2; ++sgi) {
    const float* kp = sgi ? it.k1 : it.k0;
    const float* vp = sgi ? it.v1 : it.v0;
    const int nkeys = sgi ? it.n1 : it.n0;
    const bool masked = sgi ? true : it.masked0;
    if (nkeys <= 0) continue;
    load_tile(kp, vp, nkeys, 0);
    for (int kb = 0; kb < nkeys; kb += KT) {
      lds_barrier();           // the previous tile's LDS reads are complete
      store_tile();
      if (kb + KT < nkeys) load_tile(kp, vp, nkeys, kb + KT);
      lds_barrier();
      process_tile(kb, nkeys, masked);
    }
  }

  write_partial_f32<D, 2>(a, it.slot, valid, orow, m_run, l_run, o, jj);
}

// Merge the slots of every output row: out = sum_s w_s o_s / sum_s w_s l_s,
// w_s = 2^(m_s - max_s m_s); empty slots (m_s = -inf) drop out.  Each lane
// takes VPL consecutive record positions of a row -- 4 float32 (16 bytes),
// or 8 int16 of a compact record (16 bytes, scaled by the record's c) --
// so a row's slot is one contiguous read.  In a compact record, position
// 32 k + 8 jj + 4 e + i holds dim 16 (2 k + e) + 4 jj + i, so a lane's
// positions p .. p + 7 are the dims of two groups of four.  SW groups of the row's
// lanes split its slots (SW = 1 for many rows and few slots, 8 for few
// rows and many slots); each group takes its slots four at a time with
// every load of the batch issued first, rescaling its running sums when a
// batch raises the max, and the groups merge through LDS.
template <typename T, int D, int SW, bool kCompact>
__global__ __launch_bounds__(256) void attn_combine_kernel(const AttnArgs a) {
  constexpr int VPL = kCompact ? 8 : 4;   // record values per lane
  constexpr int NV = VPL / 4;              // groups of four
  constexpr int LPR = D / VPL;             // lanes per row and slot group
  constexpr int RPB = 256 / (LPR * SW);    // rows per workgroup
  constexpr int B = 4;
  __shared__ float red_m[SW > 1 ? 256 : 1], red_l[SW > 1 ? 256 : 1];
  __shared__ f32x4 red_o[NV][SW > 1 ? 256 : 1];
  const int t = threadIdx.x;
  // the fields every lane needs, loaded in one burst (as in the partial kernel;
  // measured: section decode +1.4%)
  asm volatile("" ::"s"(a.rows_total), "s"(a.n_slots), "s"(a.ws_o), "s"(a.ws_ml), "s"(a.out), "s"(a.xmap));
  const int sub = (t / LPR) % SW;
  int row;
  bool live;
  if (a.xmap) {
    // workgroup 8 k + x: block k % comb_wpr of local row tile k / comb_wpr of
    // XCD x, whose records that XCD's partial workgroups wrote
    const int k = blockIdx.x >> 3;
    const int jl = fast_div(k, a.dv_comb);
    const int rt = xmap_tile(a, blockIdx.x & 7, jl);
    const int grp = rt < 0 ? 0 : fast_div(rt, a.dv_mt_prefix);
    const int m = (rt - grp * a.n_mt_prefix) * a.tile_rows + (k - jl * a.comb_wpr) * RPB + t / (LPR * SW);
    live = rt >= 0 && m < a.R * a.group;
    const int s = fast_div(grp, a.dv_hkv);
    const int r = fast_div(m, a.dv_group);
    row = live ? (s * a.R + r) * a.Hq + (grp - s * a.Hkv) * a.group + (m - r * a.group) : 0;
  } else {
    row = blockIdx.x * RPB + t / (LPR * SW);
    live = row < a.rows_total;
  }
  const int pos = (t % LPR) * VPL;          // record position of this lane's first value
  int dim[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int q = pos + 4 * v;
    dim[v] = kCompact ? 32 * (q / 32) + 16 * ((q % 8) / 4) + 4 * ((q % 32) / 8) : q;
  }
  float wm = kNegInf, wl = 0.f;
  f32x4 acc[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = sub; live && s0 < a.n_slots; s0 += B * SW) {
    float2 ml[B];
    f32x4 ov[B][NV];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int s = s0 + u * SW;
      ml[u] = float2{kNegInf, 0.f};
#pragma unroll
      for (int v = 0; v < NV; ++v) ov[u][v] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (s < a.n_slots) {
        const long long prow = (long long)s * a.rows_total + row;
        if constexpr (kCompact) {
          const f32x4 r = static_cast<const f32x4*>(a.ws_ml)[prow];
          const u32x4 h = *reinterpret_cast<const u32x4*>(static_cast<const int16_t*>(a.ws_o) + prow * D + pos);
          ml[u] = float2{r[0], r[1]};
#pragma unroll
          for (int v = 0; v < NV; ++v)
            ov[u][v] = f32x4{(float)(int16_t)(h[2 * v] & 0xffffu), (float)(int16_t)(h[2 * v] >> 16),
                             (float)(int16_t)(h[2 * v + 1] & 0xffffu), (float)(int16_t)(h[2 * v + 1] >> 16)} * r[2];
        } else {
          ml[u] = static_cast<const float2*>(a.ws_ml)[prow];
          ov[u][0] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.ws_o) + prow * D + pos);
        }
      }
    }
    float bm = kNegInf;
#pragma unroll
    for (int u = 0; u < B; ++u) bm = fmaxf(bm, ml[u].x);
    const float nm = fmaxf(wm, bm);
    if (nm == kNegInf) continue;
    const float sc = __builtin_amdgcn_exp2f(wm - nm);
    wl *= sc;
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[v] *= sc;
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const float w = ml[u].x == kNegInf ? 0.f : __builtin_amdgcn_exp2f(ml[u].x - nm);
      wl += w * ml[u].y;
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[v] += w * ov[u][v];
    }
    wm = nm;
  }
  if constexpr (SW > 1) {
    red_m[t] = wm;
    red_l[t] = wl;
#pragma unroll
    for (int v = 0; v < NV; ++v) red_o[v][t] = acc[v];
    __syncthreads();
    if (sub != 0 || !live) return;
    float M = kNegInf;
#pragma unroll
    for (int g = 0; g < SW; ++g) M = fmaxf(M, red_m[t + g * LPR]);
    wl = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (M != kNegInf) {
#pragma unroll
      for (int g = 0; g < SW; ++g) {
        const float mg = red_m[t + g * LPR];
        const float f = mg == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mg - M);
        wl += f * red_l[t + g * LPR];
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] += f * red_o[v][t + g * LPR];
      }
    }
  } else {
    if (!live) return;
  }
  const float inv = wl > 0.f ? 1.f / wl : 0.f;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const f32x4 x = acc[v] * inv;
    T* out = static_cast<T*>(a.out) + (long long)row * D + dim[v];
    if constexpr (sizeof(T) == 2) {
      uint16_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const __bf16 b = (__bf16)x[e];
        h[e] = __builtin_bit_cast(uint16_t, b);
      }
      *reinterpret_cast<uint2*>(out) = uint2{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16)};
    } else {
      *reinterpret_cast<f32x4*>(out) = x;
    }
  }
}

// partial workgroups: one per item, or under the XCD-aligned mapping 8 per
// (local row tile, slot) with padding
inline int partial_grid(const AttnArgs& a) {
  return a.xmap ? 8 * a.units_per_xcd * a.unit_tiles * a.n_slots : a.n_items;
}

// kDyn: the device-resident plan's instantiations (a.dyn set); the ordinary
// ones never look at it
template <int D, bool kDyn>
hipError_t launch_partial_bf16(const AttnArgs& a, hipStream_t stream) {
  if constexpr (D == 128 && !kDyn) {
    if (a.fork_rows) {
      hipLaunchKernelGGL((attn_fork_rows_kernel<128>), dim3(a.S * a.Hkv * 2 * a.n_splits), dim3(2 * kForkRG * 64),
                         kForkLdsBytes, stream, a);
      return hipGetLastError();
    }
  }
  if (a.cols == 1)
    hipLaunchKernelGGL((attn_partial_bf16_kernel<D, 4, 1, kDyn>), dim3(partial_grid(a)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_partial_bf16_kernel<D, 4, 2, kDyn>), dim3(partial_grid(a)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool kDyn>
hipError_t launch_partial_f32(const AttnArgs& a, hipStream_t stream) {
  if (a.waves == 2)
    hipLaunchKernelGGL((attn_partial_f32_kernel<D, 2, kDyn>), dim3(partial_grid(a)), dim3(128), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_partial_f32_kernel<D, 4, kDyn>), dim3(partial_grid(a)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <bool kDyn>
hipError_t launch_partial(const AttnArgs& a, int dtype, hipStream_t stream) {
  if (dtype == BC_BF16)
    return a.D == 128 ? launch_partial_bf16<128, kDyn>(a, stream) : launch_partial_bf16<64, kDyn>(a, stream);
  return a.D == 128 ? launch_partial_f32<128, kDyn>(a, stream) : launch_partial_f32<64, kDyn>(a, stream);
}

template <typename T, int D, int SW, bool kCompact>
hipError_t launch_combine_rows(const AttnArgs& a, hipStream_t stream) {
  constexpr int rows_per_block = 256 / (D / (kCompact ? 8 : 4) * SW);
  if (!a.xmap) {
    hipLaunchKernelGGL((attn_combine_kernel<T, D, SW, kCompact>),
                       dim3((a.rows_total + rows_per_block - 1) / rows_per_block), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  // a row tile's rows in whole workgroups (tile_rows is a multiple of the
  // rows per workgroup)
  AttnArgs b = a;
  b.comb_wpr = a.tile_rows / rows_per_block;
  b.dv_comb = make_fastdiv(b.comb_wpr);
  hipLaunchKernelGGL((attn_combine_kernel<T, D, SW, kCompact>),
                     dim3(8 * a.units_per_xcd * a.unit_tiles * b.comb_wpr), dim3(256), 0, stream, b);
  return hipGetLastError();
}

template <typename T, int D, int SW>
hipError_t launch_combine_sw(const AttnArgs& a, hipStream_t stream) {
  if (sizeof(T) == 2 && a.compact) return launch_combine_rows<T, D, SW, sizeof(T) == 2>(a, stream);
  return launch_combine_rows<T, D, SW, false>(a, stream);
}

// slot groups per row: with few rows, enough that each group's slots are
// one batch of loads (4), up to 8 groups; walking more slots in one group
// serialises a round trip per batch (measured: 2048 rows of 13 slots took
// 5.1 us with one group, 3.8 us with four).  With many rows the other
// waves hide those round trips and the groups' LDS merge only costs (9216
// rows of 7 slots: 4.8 us with one group, 5.8 us with two).
template <typename T, int D>
hipError_t launch_combine_typed(const AttnArgs& a, hipStream_t stream) {
  const int groups = a.rows_total <= 4096 ? (a.n_slots + 3) / 4 : 1;
  if (groups > 4) return launch_combine_sw<T, D, 8>(a, stream);
  if (groups > 2) return launch_combine_sw<T, D, 4>(a, stream);
  if (groups > 1) return launch_combine_sw<T, D, 2>(a, stream);
  return launch_combine_sw<T, D, 1>(a, stream);
}

}  // namespace

hipError_t launch_attn_partial(const AttnArgs& a, int dtype, hipStream_t stream) {
  return a.dyn ? launch_partial<true>(a, dtype, stream) : launch_partial<false>(a, dtype, stream);
}

hipError_t launch_attn_combine(const AttnArgs& a, int dtype, hipStream_t stream) {
  if (a.direct) return hipSuccess;   // the partial pass wrote the output
  if (dtype == BC_BF16)
    return a.D == 128 ? launch_combine_typed<bf16_t, 128>(a, stream) : launch_combine_typed<bf16_t, 64>(a, stream);
  return a.D == 128 ? launch_combine_typed<float, 128>(a, stream) : launch_combine_typed<float, 64>(a, stream);
}

}  // namespace bc
