// Internal declarations shared by the host entry points (bc_api.cpp) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bc.h"

namespace bc {

// ---------------------------------------------------------------- attention
constexpr int kAttnWaves = 4;             // waves per workgroup
constexpr int kAttnRowsPerWave = 32;      // query rows per wave (2 MFMA column tiles)
constexpr int kAttnTileRows = kAttnWaves * kAttnRowsPerWave;
constexpr int kAttnKeyTile = 64;          // keys staged through LDS per iteration

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
  float* ws_o;         // [n_slots][rows_total][D] unnormalised partial outputs
  float2* ws_ml;       // [n_slots][rows_total] (running max in log2 units, sum)
  float scale_log2;    // softmax scale * log2(e)
  int S, R, Hq, Hkv, group, D;
  int fork;            // 1: one shared prefix for all S rollouts + private caches
  int causal;          // bc_mask
  int n_splits;        // prefix chunks P; slot P holds private + active keys
  int n_slots;         // P + 1
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
};

hipError_t launch_attn(const AttnArgs& a, int dtype, hipStream_t stream);

// -------------------------------------------------------------- commit
hipError_t launch_commit(void* cache, const void* blk, int dtype, int Hkv, int D,
                         long long seq_stride, long long head_stride, int start, int n_rows,
                         hipStream_t stream);

// -------------------------------------------------------------- vocab scans
constexpr int kScanThreads = 256;
constexpr int kScanVecPerThread = 8;                                // float4 per thread
constexpr int kScanChunk = kScanThreads * kScanVecPerThread * 4;    // 8192 logits

struct ScanPartial { float m; int a; float s; int pad; };

inline int scan_chunks(int vocab) { return (vocab + kScanChunk - 1) / kScanChunk; }

struct UnmaskArgs {
  const float* logits;
  int n_rows, vocab, n_chunks, n_blk;
  uint8_t* masked;
  int* tokens;
  float* conf;
  int* n_commit;
  ScanPartial* part;   // [n_rows][n_chunks]
  float threshold;
  int blk_off[BC_MAX_BLOCKS + 1];
  int mode[BC_MAX_BLOCKS];
  int n_div[BC_MAX_BLOCKS];
};

hipError_t launch_unmask(const UnmaskArgs& a, hipStream_t stream);

struct VerifyArgs {
  const float* logits;
  int n_seq, n_lrows, vocab, n_chunks, m;
  const int* draft;
  const uint8_t* fixed;
  const int* first;
  int* accept_len;
  int* bonus;
  ScanPartial* part;   // [n_seq * n_lrows][n_chunks]
};

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);

}  // namespace bc
