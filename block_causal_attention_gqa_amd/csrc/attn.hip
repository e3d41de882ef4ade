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
// stream serves all `group` query heads.  A workgroup (2 or 4 waves x 32
// rows) takes one row tile against one key range and writes an unnormalised
// partial (running max, sum, output) to its slot:
//   * prefix items: slot p < P covers chunk p of the committed prefix; under
//     a fork the tile runs over the rows of ALL rollouts, so the shared prefix
//     is streamed once per tile instead of once per rollout;
//   * active items: slot P covers the rollout's private keys plus the active
//     keys, where the block predicate applies.  The predicate is never stored:
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
// registers.  V^T is staged in LDS transposed (V is stored [key][dim] in HBM).
// The per-column softmax scalars (max, rescale) are per lane.  fp32 inputs
// use v_mfma_f32_16x16x4_f32 with the same structure.

#include <type_traits>

#include "bc_internal.h"

namespace bc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;   // raw bf16 storage

constexpr float kNegInf = -__builtin_huge_valf();

template <typename T, int D> struct Cfg;
template <int D> struct Cfg<bf16_t, D> {
  static constexpr int KP = D + 8;                 // K row pitch (elements)
  static constexpr int VP = kAttnKeyTile + 8;      // V^T row pitch (elements)
  static constexpr int K_ELEMS = kAttnKeyTile * KP;
  static constexpr int V_ELEMS = D * VP;
};
template <int D> struct Cfg<float, D> {
  static constexpr int KP = D + 4;
  static constexpr int VP = D + 4;                 // V kept [key][dim]
  static constexpr int K_ELEMS = kAttnKeyTile * KP;
  static constexpr int V_ELEMS = kAttnKeyTile * VP;
};

__device__ inline float wave_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// x when keep, else zero -- component-wise, so no aggregate select (which
// the compiler lowers through stack memory)
__device__ inline uint4 keep_or_zero(bool keep, const uint4& x) {
  return uint4{keep ? x.x : 0u, keep ? x.y : 0u, keep ? x.z : 0u, keep ? x.w : 0u};
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

// position inside the 64-key tile of the value held in C-register i of tile t
template <typename T>
__device__ inline int key_pos(int t, int jj, int i) {
  if constexpr (sizeof(T) == 2) return 32 * (t >> 1) + 8 * jj + 4 * (t & 1) + i;
  else return 16 * t + 4 * jj + i;
}

template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_partial_kernel(const AttnArgs a) {
  using C = Cfg<T, D>;
  constexpr int NT = NW * 64;                 // threads
  constexpr int kTileRows = NW * kAttnRowsPerWave;
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int KT = kAttnKeyTile;
  __shared__ __attribute__((aligned(16))) T k_lds[C::K_ELEMS];
  __shared__ __attribute__((aligned(16))) T v_lds[C::V_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, jj = lane >> 4;

  // ---- which item this workgroup computes
  const int item = xcd_remap(blockIdx.x, a.n_items);
  const bool is_prefix = item < a.n_prefix_items;
  int g, mt, slot, s_item, rows_in_group, key_begin, key_end, lv = 0;
  const T* kbase = nullptr;   // prefix items: row 0 of the (seq, kv head) cache
  const T* vbase = nullptr;
  if (is_prefix) {
    mt = item % a.n_mt_prefix;
    const int rest = item / a.n_mt_prefix;
    slot = rest % a.n_splits;
    const int grp = rest / a.n_splits;
    int ps;
    if (a.fork) { g = grp; s_item = -1; ps = 0; rows_in_group = a.S * a.R * a.group; }
    else { g = grp % a.Hkv; s_item = grp / a.Hkv; ps = s_item; rows_in_group = a.R * a.group; }
    key_begin = slot * a.chunk[ps];
    key_end = min(a.prefix_len[ps], key_begin + a.chunk[ps]);
    const long long off = ps * a.p_seq_stride + g * a.p_head_stride;
    kbase = static_cast<const T*>(a.pk) + off;
    vbase = static_cast<const T*>(a.pv) + off;
  } else {
    const int it = item - a.n_prefix_items;
    mt = it % a.n_mt_active;
    const int rest = it / a.n_mt_active;
    g = rest % a.Hkv;
    s_item = rest / a.Hkv;
    slot = a.n_splits;
    rows_in_group = a.R * a.group;
    lv = a.fork ? a.priv_len[s_item] : 0;
    key_begin = 0;
    key_end = lv + a.R;
  }

  // ---- this lane's two query columns
  bool valid[2];
  int orow[2], lim[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int m = mt * kTileRows + wave * kAttnRowsPerWave + c * 16 + n;
    valid[c] = m < rows_in_group;
    int s = s_item, rem = m;
    if (s_item < 0) { s = m / (a.R * a.group); rem = m - s * (a.R * a.group); }
    const int r = rem / a.group, hh = rem - r * a.group;
    orow[c] = valid[c] ? (s * a.R + r) * a.Hq + g * a.group + hh : 0;
    int l = r + 1;
    if (!a.causal) {
      l = a.R;
      for (int b = 0; b < a.n_blk; ++b)
        if (r < a.blk_off[b + 1]) { l = a.blk_off[b + 1]; break; }
    }
    lim[c] = l;
  }
  const int s_act = s_item;   // active items: the sequence whose private/active keys are read

  // ---- Q^T operand, resident for the whole item
  const T* q = static_cast<const T*>(a.q);
  constexpr int QK = kBf16 ? D / 32 : D / 4;
  using QOp = typename std::conditional<kBf16, bf16x8, float>::type;
  QOp qop[2][QK];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int kk = 0; kk < QK; ++kk) {
      if constexpr (kBf16) {
        bf16x8 z = {};
        qop[c][kk] = valid[c] ? *reinterpret_cast<const bf16x8*>(q + (long long)orow[c] * D + 32 * kk + 8 * jj) : z;
      } else {
        qop[c][kk] = valid[c] ? q[(long long)orow[c] * D + 4 * kk + jj] : 0.f;
      }
    }

  float m_run[2] = {kNegInf, kNegInf};
  float l_run[2] = {0.f, 0.f};
  f32x4 o[2][D / 16];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[c][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- the item's keys as at most two contiguous segments, each read from
  // one base pointer: the prefix chunk; or the rollout's private keys, then
  // the active keys (the only segment the block predicate applies to).
  const T *seg0_k, *seg0_v, *seg1_k = nullptr, *seg1_v = nullptr;
  int seg0_n, seg1_n = 0;
  bool seg0_masked;
  if (is_prefix) {
    seg0_k = kbase + (long long)key_begin * D;
    seg0_v = vbase + (long long)key_begin * D;
    seg0_n = max(0, key_end - key_begin);
    seg0_masked = false;
  } else {
    const long long act_off = (long long)(s_act * a.Hkv + g) * a.R * D;
    const T* ak = static_cast<const T*>(a.ak) + act_off;
    const T* av = static_cast<const T*>(a.av) + act_off;
    if (lv > 0) {
      const long long prv_off = s_act * a.v_seq_stride + g * a.v_head_stride;
      seg0_k = static_cast<const T*>(a.vk) + prv_off;
      seg0_v = static_cast<const T*>(a.vv) + prv_off;
      seg0_n = lv;
      seg0_masked = false;
      seg1_k = ak;
      seg1_v = av;
      seg1_n = a.R;
    } else {
      seg0_k = ak;
      seg0_v = av;
      seg0_n = a.R;
      seg0_masked = true;
    }
  }

  // ---- register staging of one key tile: the next tile's global loads are
  // issued before the current tile is computed, so HBM latency is paid once.
  // Loads are clamped to the segment's last key and zeroed past its end, so
  // they need no branches.
  constexpr int CPR = kBf16 ? D / 8 : D / 4;           // 16-byte units per key row
  constexpr int EPU = kBf16 ? 8 : 4;                   // elements per 16-byte unit
  constexpr int NK = (KT * CPR + NT - 1) / NT;         // K units per thread
  constexpr int NVQ = ((KT / 4) * CPR + NT - 1) / NT;  // bf16: 4-key quads per thread
  constexpr int NV = kBf16 ? 4 * NVQ : NK;             // V units per thread
  uint4 kreg[NK], vreg[NV];

  auto load_tile = [&](const T* kp, const T* vp, int nkeys, int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const int idx = tid + NT * u;
      const int kr = idx / CPR, cc = idx - kr * CPR;
      const int key = kb + kr;
      const long long off = (long long)min(key, nkeys - 1) * D + EPU * cc;
      const uint4 kx = *reinterpret_cast<const uint4*>(kp + off);
      kreg[u] = keep_or_zero(key < nkeys, kx);
      if constexpr (!kBf16) {
        const uint4 vx = *reinterpret_cast<const uint4*>(vp + off);
        vreg[u] = keep_or_zero(key < nkeys, vx);
      }
    }
    if constexpr (kBf16) {
#pragma unroll
      for (int u = 0; u < NVQ; ++u) {
        const int idx = tid + NT * u;
        const int qd = idx % (KT / 4), cc = idx / (KT / 4);
        const bool in_tile = idx < (KT / 4) * CPR;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb + 4 * qd + i;
          const long long off = (long long)min(key, nkeys - 1) * D + 8 * min(cc, CPR - 1);
          const uint4 vx = *reinterpret_cast<const uint4*>(vp + off);
          vreg[4 * u + i] = keep_or_zero(in_tile && key < nkeys, vx);
        }
      }
    }
  };

  auto store_tile = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const int idx = tid + NT * u;
      if (idx >= KT * CPR) continue;
      const int kr = idx / CPR, cc = idx - kr * CPR;
      if constexpr (kBf16) {
        *reinterpret_cast<uint4*>(&k_lds[kr * C::KP + 8 * cc]) = kreg[u];
      } else {
        *reinterpret_cast<uint4*>(&k_lds[kr * C::KP + 4 * cc]) = kreg[u];
        *reinterpret_cast<uint4*>(&v_lds[kr * C::VP + 4 * cc]) = vreg[u];
      }
    }
    if constexpr (kBf16) {
      // V transposed: 4 consecutive keys x 8 dims -> 8 rows of V^T, 4 keys each
#pragma unroll
      for (int u = 0; u < NVQ; ++u) {
        const int idx = tid + NT * u;
        if (idx >= (KT / 4) * CPR) continue;
        const int qd = idx % (KT / 4), cc = idx / (KT / 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t sh = (e & 1) * 16;
          const int w = e >> 1;
          auto pick = [&](const uint4& x) -> uint32_t {
            const uint32_t word = w == 0 ? x.x : w == 1 ? x.y : w == 2 ? x.z : x.w;
            return (word >> sh) & 0xffffu;
          };
          uint2 packed;
          packed.x = pick(vreg[4 * u]) | (pick(vreg[4 * u + 1]) << 16);
          packed.y = pick(vreg[4 * u + 2]) | (pick(vreg[4 * u + 3]) << 16);
          *reinterpret_cast<uint2*>(&v_lds[(8 * cc + e) * C::VP + 4 * qd]) = packed;
        }
      }
    }
  };

  // one 64-key tile: keys kb .. kb + 63 of a segment of nkeys keys
  auto process_tile = [&](int kb, int nkeys, bool masked) __attribute__((always_inline)) {
    // ---- S^T = K Q^T for 4 tiles of 16 keys x 2 column tiles
    f32x4 st[2][4];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t) st[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (kBf16) {
        // all A operands of the 16-key tile first, so the LDS reads overlap
        const int krow = 32 * (t >> 1) + 8 * (n >> 2) + 4 * (t & 1) + (n & 3);
        bf16x8 ka[D / 32];
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
          ka[kk] = *reinterpret_cast<const bf16x8*>(&k_lds[krow * C::KP + 32 * kk + 8 * jj]);
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
          for (int c = 0; c < 2; ++c)
            st[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kk], qop[c][kk], st[c][t], 0, 0, 0);
      } else {
#pragma unroll
        for (int kk = 0; kk < D / 4; ++kk) {
          const float ka = k_lds[(16 * t + n) * C::KP + 4 * kk + jj];
#pragma unroll
          for (int c = 0; c < 2; ++c)
            st[c][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka, qop[c][kk], st[c][t], 0, 0, 0);
        }
      }
    }

    // ---- online softmax, one query column per lane and column tile
    // a tile inside an unmasked segment is fully visible: no predicate.
    // Scores stay unscaled here (scale > 0 keeps their order); the scale is
    // applied inside the exponent, p = 2^(x * scale * log2 e - m).
    const bool full_tile = !masked && kb + KT <= nkeys;
    const float sl2 = a.scale_log2;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float tmax = kNegInf;
      if (full_tile) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, st[c][t][i]);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kb + key_pos<T>(t, jj, i);
            const bool vis = key < nkeys && (!masked || key < lim[c]);
            const float x = vis ? st[c][t][i] : kNegInf;
            st[c][t][i] = x;
            tmax = fmaxf(tmax, x);
          }
      }
      tmax = fmaxf(tmax, wave_xor(tmax, 16));
      tmax = fmaxf(tmax, wave_xor(tmax, 32));
      const float mnew = fmaxf(m_run[c], tmax * sl2);        // running max, scaled
      const float muse = mnew == kNegInf ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(m_run[c] - muse);
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
      if (__any(alpha != 1.f)) {   // wave-uniform: skip when no column's max moved
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[c][dt] *= alpha;
      }
    }

    // ---- O^T += V^T P^T
    if constexpr (kBf16) {
      bf16x8 pb[2][2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pb[c][ks][e] = (__bf16)st[c][2 * ks][e];
            pb[c][ks][e + 4] = (__bf16)st[c][2 * ks + 1][e];
          }
#pragma unroll
      for (int dt0 = 0; dt0 < D / 16; dt0 += 4) {
        // A operands of four 16-dim tiles first, then their MFMAs
        bf16x8 va[4][2];
#pragma unroll
        for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            va[d4][ks] = *reinterpret_cast<const bf16x8*>(
                &v_lds[(16 * (dt0 + d4) + n) * C::VP + 32 * ks + 8 * jj]);
#pragma unroll
        for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int c = 0; c < 2; ++c)
              o[c][dt0 + d4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[d4][ks], pb[c][ks], o[c][dt0 + d4], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float va = v_lds[(16 * t + 4 * jj + i) * C::VP + 16 * dt + n];
#pragma unroll
            for (int c = 0; c < 2; ++c)
              o[c][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va, st[c][t][i], o[c][dt], 0, 0, 0);
          }
    }
  };

  // ---- stream the segments' key tiles through LDS (one code path for both)
  for (int sgi = 0; sgi < 2; ++sgi) {
    const T* kp = sgi ? seg1_k : seg0_k;
    const T* vp = sgi ? seg1_v : seg0_v;
    const int nkeys = sgi ? seg1_n : seg0_n;
    const bool masked = sgi ? true : seg0_masked;
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

  // ---- write this item's partial
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    float l = l_run[c];
    l += wave_xor(l, 16);
    l += wave_xor(l, 32);
    if (!valid[c]) continue;
    const long long prow = (long long)slot * a.rows_total + orow[c];
    if (jj == 0) a.ws_ml[prow] = float2{m_run[c], l};
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      *reinterpret_cast<f32x4*>(&a.ws_o[prow * D + 16 * dt + 4 * jj]) = o[c][dt];
  }
}

// Merge the slots of every output row: out = sum_s w_s o_s / sum_s w_s l_s,
// w_s = 2^(m_s - max_s m_s); empty slots (m_s = -inf) drop out.  One row per
// workgroup; wave w takes slots w, w + 4, ... eight at a time with every load
// of the batch issued before any is used, rescaling online when a batch
// raises the running max; the four waves then merge through LDS.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const AttnArgs a) {
  constexpr int E = D / 64;
  constexpr int B = 8;
  __shared__ float red_o[4][D];
  __shared__ float red_m[4], red_l[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x;
  float wm = kNegInf, wl = 0.f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int s0 = wave; s0 < a.n_slots; s0 += 4 * B) {
    float2 ml[B];
    float ov[B][E];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int s = s0 + 4 * u;
      const long long prow = (long long)s * a.rows_total + row;
      ml[u] = float2{kNegInf, 0.f};
#pragma unroll
      for (int e = 0; e < E; ++e) ov[u][e] = 0.f;
      if (s < a.n_slots) {
        ml[u] = a.ws_ml[prow];
#pragma unroll
        for (int e = 0; e < E; ++e) ov[u][e] = a.ws_o[prow * D + lane + 64 * e];
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
    for (int e = 0; e < E; ++e) acc[e] *= sc;
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const float w = ml[u].x == kNegInf ? 0.f : __builtin_amdgcn_exp2f(ml[u].x - nm);
      wl += w * ml[u].y;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += w * ov[u][e];
    }
    wm = nm;
  }
  if (lane == 0) { red_m[wave] = wm; red_l[wave] = wl; }
#pragma unroll
  for (int e = 0; e < E; ++e) red_o[wave][lane + 64 * e] = acc[e];
  __syncthreads();
  if (wave != 0) return;
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w]);
  float L = 0.f, o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float f = red_m[w] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(red_m[w] - M);
    L += f * red_l[w];
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] += f * red_o[w][lane + 64 * e];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  T* out = static_cast<T*>(a.out) + (long long)row * D;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float v = o[e] * inv;
    if constexpr (sizeof(T) == 2) {
      const __bf16 b = (__bf16)v;
      out[lane + 64 * e] = *reinterpret_cast<const uint16_t*>(&b);
    } else {
      out[lane + 64 * e] = v;
    }
  }
}

template <typename T, int D>
hipError_t launch_partial_typed(const AttnArgs& a, hipStream_t stream) {
  if (a.waves == 2)
    hipLaunchKernelGGL((attn_partial_kernel<T, D, 2>), dim3(a.n_items), dim3(128), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_partial_kernel<T, D, 4>), dim3(a.n_items), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_combine_typed(const AttnArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((attn_combine_kernel<T, D>), dim3(a.rows_total), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_partial(const AttnArgs& a, int dtype, hipStream_t stream) {
  if (dtype == BC_BF16)
    return a.D == 128 ? launch_partial_typed<bf16_t, 128>(a, stream) : launch_partial_typed<bf16_t, 64>(a, stream);
  return a.D == 128 ? launch_partial_typed<float, 128>(a, stream) : launch_partial_typed<float, 64>(a, stream);
}

hipError_t launch_attn_combine(const AttnArgs& a, int dtype, hipStream_t stream) {
  if (dtype == BC_BF16)
    return a.D == 128 ? launch_combine_typed<bf16_t, 128>(a, stream) : launch_combine_typed<bf16_t, 64>(a, stream);
  return a.D == 128 ? launch_combine_typed<float, 128>(a, stream) : launch_combine_typed<float, 64>(a, stream);
}

}  // namespace bc
