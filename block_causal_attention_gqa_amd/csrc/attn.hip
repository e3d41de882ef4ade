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
// stream serves all `group` query heads.  A workgroup (4 waves x 32 rows)
// takes one 128-row tile against one key range and writes an unnormalised
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

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_partial_kernel(const AttnArgs a) {
  using C = Cfg<T, D>;
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
    const int m = mt * kAttnTileRows + wave * kAttnRowsPerWave + c * 16 + n;
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

  // row pointer of key `key` of this item (K or V)
  auto key_row = [&](int key, bool want_v) -> const T* {
    if (is_prefix) return (want_v ? vbase : kbase) + (long long)key * D;
    if (key < lv) {
      const T* base = static_cast<const T*>(want_v ? a.vv : a.vk);
      return base + s_act * a.v_seq_stride + g * a.v_head_stride + (long long)key * D;
    }
    const T* base = static_cast<const T*>(want_v ? a.av : a.ak);
    return base + ((long long)(s_act * a.Hkv + g) * a.R + (key - lv)) * D;
  };

  for (int kb = key_begin; kb < key_end; kb += KT) {
    __syncthreads();
    // ---- stage K (and V) of keys kb .. kb + 63 in LDS; keys past the range are zero
    if constexpr (kBf16) {
      constexpr int CPR = D / 8;   // 16-byte chunks per row
      for (int idx = tid; idx < KT * CPR; idx += 256) {
        const int kr = idx / CPR, cc = idx - kr * CPR;
        const int key = kb + kr;
        uint4 val = {0u, 0u, 0u, 0u};
        if (key < key_end) val = *reinterpret_cast<const uint4*>(key_row(key, false) + 8 * cc);
        *reinterpret_cast<uint4*>(&k_lds[kr * C::KP + 8 * cc]) = val;
      }
      // V transposed: each thread takes 4 consecutive keys x 8 dims
      for (int idx = tid; idx < (KT / 4) * CPR; idx += 256) {
        const int qd = idx % (KT / 4), cc = idx / (KT / 4);
        uint4 v4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb + 4 * qd + i;
          v4[i] = uint4{0u, 0u, 0u, 0u};
          if (key < key_end) v4[i] = *reinterpret_cast<const uint4*>(key_row(key, true) + 8 * cc);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t sh = (e & 1) * 16;
          const int w = e >> 1;
          auto pick = [&](const uint4& x) -> uint32_t {
            const uint32_t word = w == 0 ? x.x : w == 1 ? x.y : w == 2 ? x.z : x.w;
            return (word >> sh) & 0xffffu;
          };
          uint2 packed;
          packed.x = pick(v4[0]) | (pick(v4[1]) << 16);
          packed.y = pick(v4[2]) | (pick(v4[3]) << 16);
          *reinterpret_cast<uint2*>(&v_lds[(8 * cc + e) * C::VP + 4 * qd]) = packed;
        }
      }
    } else {
      constexpr int CPR = D / 4;
      for (int idx = tid; idx < KT * CPR; idx += 256) {
        const int kr = idx / CPR, cc = idx - kr * CPR;
        const int key = kb + kr;
        float4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
        if (key < key_end) {
          kv = *reinterpret_cast<const float4*>(key_row(key, false) + 4 * cc);
          vv = *reinterpret_cast<const float4*>(key_row(key, true) + 4 * cc);
        }
        *reinterpret_cast<float4*>(&k_lds[kr * C::KP + 4 * cc]) = kv;
        *reinterpret_cast<float4*>(&v_lds[kr * C::VP + 4 * cc]) = vv;
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for 4 tiles of 16 keys x 2 column tiles
    f32x4 st[2][4];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t) st[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (kBf16) {
        const int krow = 32 * (t >> 1) + 8 * (n >> 2) + 4 * (t & 1) + (n & 3);
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&k_lds[krow * C::KP + 32 * kk + 8 * jj]);
#pragma unroll
          for (int c = 0; c < 2; ++c)
            st[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qop[c][kk], st[c][t], 0, 0, 0);
        }
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
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float tmax = kNegInf;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb + key_pos<T>(t, jj, i);
          const bool vis = key < key_end && (is_prefix || key < lv || key - lv < lim[c]);
          const float x = vis ? st[c][t][i] * a.scale_log2 : kNegInf;
          st[c][t][i] = x;
          tmax = fmaxf(tmax, x);
        }
      tmax = fmaxf(tmax, wave_xor(tmax, 16));
      tmax = fmaxf(tmax, wave_xor(tmax, 32));
      const float mnew = fmaxf(m_run[c], tmax);
      const float muse = mnew == kNegInf ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(m_run[c] - muse);
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(st[c][t][i] - muse);
          st[c][t][i] = p;
          psum += p;
        }
      l_run[c] = l_run[c] * alpha + psum;
      m_run[c] = mnew;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[c][dt] *= alpha;
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
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(&v_lds[(16 * dt + n) * C::VP + 32 * ks + 8 * jj]);
#pragma unroll
          for (int c = 0; c < 2; ++c)
            o[c][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[c][ks], o[c][dt], 0, 0, 0);
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
// w_s = 2^(m_s - max_s m_s); empty slots (m_s = -inf) drop out.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows_total) return;
  float mx = kNegInf;
  for (int s = 0; s < a.n_slots; ++s) mx = fmaxf(mx, a.ws_ml[(long long)s * a.rows_total + row].x);
  constexpr int E = D / 64;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float L = 0.f;
  for (int s = 0; s < a.n_slots; ++s) {
    const long long prow = (long long)s * a.rows_total + row;
    const float2 ml = a.ws_ml[prow];
    if (ml.x == kNegInf) continue;
    const float w = __builtin_amdgcn_exp2f(ml.x - mx);
    L += w * ml.y;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += w * a.ws_o[prow * D + lane + 64 * e];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  T* out = static_cast<T*>(a.out) + (long long)row * D;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float v = acc[e] * inv;
    if constexpr (sizeof(T) == 2) {
      const __bf16 b = (__bf16)v;
      out[lane + 64 * e] = *reinterpret_cast<const uint16_t*>(&b);
    } else {
      out[lane + 64 * e] = v;
    }
  }
}

template <typename T, int D>
hipError_t launch_typed(const AttnArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((attn_partial_kernel<T, D>), dim3(a.n_items), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_combine_kernel<T, D>), dim3((a.rows_total + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, int dtype, hipStream_t stream) {
  if (dtype == BC_BF16) return a.D == 128 ? launch_typed<bf16_t, 128>(a, stream) : launch_typed<bf16_t, 64>(a, stream);
  return a.D == 128 ? launch_typed<float, 128>(a, stream) : launch_typed<float, 64>(a, stream);
}

}  // namespace bc
