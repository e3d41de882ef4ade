// Internal declarations shared by the host entry points (api.hip) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bc.h"   // include/bc.h (the build passes -I include)

namespace bc {

// Division by a launch-invariant divisor d >= 1 with one multiply-high: for
// 0 <= n < 2^31, n / d = (umulhi(n, mul) + n) >> shift, with shift =
// ceil(log2 d) and mul = floor(2^32 (2^shift - d) / d) + 1 (division by
// invariant integers using multiplication, Granlund and Montgomery 1994).
// The kernels split item and row indices this way instead of through the
// long integer-division sequence, which sits before their first loads.
struct FastDiv {
  uint32_t mul, shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  return FastDiv{(uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1), s};
}

__device__ inline int fast_div(int n, FastDiv f) {
  return (int)((__umulhi((uint32_t)n, f.mul) + (uint32_t)n) >> f.shift);
}

// ---------------------------------------------------------------- attention
constexpr int kAttnKeyTile = 64;          // keys staged through LDS per iteration
constexpr int kCompactRows = 1024;        // bf16 calls with at least this many output rows use compact partials
constexpr int kForkTileRows = 96;         // rows per row tile of the fork's row-tile form (half a rollout's rows)

// The next step of a device-resident pipelined decode (bc_dev_plan, see
// include/bc.h), written by the schedule kernel and read by the step's kernels.
using DevPlan = bc_dev_plan;
struct UnmaskArgs;

struct AttnArgs {
  const void* q;       // [S][R][Hq][D]
  void* out;           // [S][R][Hq][D]
  const void* pk;      // prefix cache [Sp][Hkv][cap][D]
  const void* pv;
  long long p_seq_stride, p_head_stride;   // elements
  const void* vk;      // private cache (fork) [S][Hkv][capv][D] or null
  const void* vv;
  long long v_seq_stride, v_head_stride;
  const void* ak;      // active K/V [S][Hkv][R][D]
  const void* av;
  // Split partials, [n_slots][rows_total] records of the unnormalised
  // output o (D values), the running max m (log2 units) and the sum l:
  //   float32:  ws_o float [..][D] = o, ws_ml float2 {m, l};
  //   compact:  ws_o int16 [..][D] = h (the writer's store order), ws_ml float4
  //             {m, l, c, 0}, with o = c h (c a power of two per record).
  void* ws_o;
  void* ws_ml;
  int compact;         // 1: compact partials (bf16 inputs only)
  float scale_log2;    // softmax scale * log2(e)
  int S, R, Hq, Hkv, group, D;
  int waves;           // waves per workgroup (2 or 4)
  int cols;            // 16-row MFMA column tiles per wave (1 or 2); a row tile is waves * cols * 16 rows
  int fork;            // 1: one shared prefix for all S rollouts + private caches
  int causal;          // bc_mask
  int n_splits;        // prefix chunks P; slot P holds private + active keys
  int n_slots;         // P + 1, or P under fold
  int fold;            // 1 (no fork): the active keys ride in the last prefix chunk's items, no slot P
  int n_mt_prefix;     // row tiles per prefix group
  int n_mt_active;     // row tiles per (seq, kv head) for the active items
  int n_prefix_items;
  int n_items;
  int rows_total;      // S * R * Hq
  int n_blk;
  int blk_off[BC_MAX_BLOCKS + 1];
  int prefix_len[BC_MAX_SEQ];
  int chunk[BC_MAX_SEQ];     // prefix keys per chunk (multiple of kAttnKeyTile)
  int priv_len[BC_MAX_SEQ];
  // n_mt_prefix, n_splits, Hkv, n_mt_active, R * group and group as FastDiv
  FastDiv dv_mt_prefix, dv_splits, dv_hkv, dv_mt_active, dv_rows, dv_group;
  // XCD-aligned mapping (calls without a fork).  Workgroup h runs on XCD
  // h % 8.  Row tiles (tile_rows rows, numbered group * n_mt_prefix + mt)
  // are taken in units of unit_tiles consecutive tiles -- a whole (sequence,
  // KV head) group when there are at least 8 groups, else one tile -- and
  // unit u belongs to XCD u % 8: every split of its row tiles (partial
  // workgroup 8 k + x, k = (local tile) * n_slots + slot) and the combine
  // workgroups of their rows (8 k + x, k = (local tile) * comb_wpr + block)
  // run there, so the combine reads records written through its own L2.
  // Workgroups past the last unit exit at once.
  int xmap;
  int tile_rows, unit_tiles, n_units, units_per_xcd;
  int comb_wpr;        // combine workgroups per row tile (set at launch)
  FastDiv dv_slots, dv_unit_tiles, dv_comb;
  // Device-resident plan (one sequence, no fork) or null: the prefix length
  // and the blocks come from it instead of prefix_len[0] / n_blk / blk_off;
  // R stays the widest step's row count; a step with no active block does
  // nothing.
  const DevPlan* dyn;
  // 1: the fork's row-tile form (one workgroup per half of a rollout's rows
  // and key split, attn_fork_rows_kernel)
  int fork_rows;
  // 1: the partial pass writes the output itself (a row-tile form with one
  // key split); the combine does nothing
  int direct;
};

// Kernel arguments of a block-bidirectional attention call without a fork,
// and of an unmask call, validated and filled as bc_attn_step and
// bc_unmask_select fill them (api.hip); BC_OK or an error.
int prepare_attn_args(const bc_kv_cache* prefix, const int32_t* prefix_len, const bc_active* a, float scale,
                      void* out, void* ws, size_t ws_bytes, AttnArgs* args);
int prepare_unmask_args(const float* logits, int32_t n_rows, int32_t vocab, const int32_t* blk_off, int32_t n_blk,
                        const int32_t* mode, const int32_t* n_div, float threshold, uint8_t* masked, int32_t* tokens,
                        int32_t* n_commit, void* ws, size_t ws_bytes, UnmaskArgs* args);

hipError_t launch_attn_partial(const AttnArgs& a, int dtype, hipStream_t stream);
hipError_t launch_attn_combine(const AttnArgs& a, int dtype, hipStream_t stream);

// -------------------------------------------------------------- commit
hipError_t launch_commit(void* k_cache, void* v_cache, const void* blk_k, const void* blk_v, int dtype,
                         int Hkv, int D, long long head_stride, int start, int n_rows, hipStream_t stream);

// -------------------------------------------------------------- vocab scans
constexpr int kScanThreads = 256;
constexpr int kScanVecPerThread = 4;                                // float4 per thread
constexpr int kScanChunk = kScanThreads * kScanVecPerThread * 4;    // 4096 logits

struct ScanPartial { float m; int a; float s; int pad; };

inline int scan_chunks(int vocab) { return (vocab + kScanChunk - 1) / kScanChunk; }

struct UnmaskArgs {
  const float* logits;
  int n_rows, vocab, n_chunks, n_blk;
  uint8_t* masked;
  int* tokens;
  float* conf;
  int* n_commit;
  const ScanPartial* part;   // [n_rows][n_chunks], left by the scan
  float threshold;
  int blk_off[BC_MAX_BLOCKS + 1];
  int mode[BC_MAX_BLOCKS];
  int n_div[BC_MAX_BLOCKS];
  // Device-resident plan or null: the blocks, modes and n come from it, and
  // masked / tokens / conf are offset by its row0.
  const DevPlan* dyn;
};

// row_mask: scan rows with row_mask[r] != 0 (all rows when null);
// with_sum: also the exp-sum (unmask) besides max / argmax.
hipError_t launch_scan(const float* logits, int n_rows, int vocab, const uint8_t* row_mask, bool with_sum,
                       ScanPartial* part, hipStream_t stream, const DevPlan* dyn = nullptr);
hipError_t launch_unmask_decide(const UnmaskArgs& a, hipStream_t stream);

struct VerifyArgs {
  const float* logits;
  int n_seq, n_lrows, vocab, n_chunks, m;
  const int* draft;
  const uint8_t* fixed;
  const int* first;
  int* accept_len;
  int* bonus;
  ScanPartial* part;   // [n_seq * n_lrows][n_chunks]
  const float* noise;  // [n_seq][n_lrows][vocab] Gumbel noise, or null (greedy)
  float inv_temperature;
};

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);

}  // namespace bc
