// Pipelined parallel decoding with the whole step loop on the host side of
// the library (Fast-dVLA reading notes, key design 4): per step the plan of
// the schedule (pipeline.hip), the caller's model outputs, the attention
// over the active blocks, the unmask with the planned modes, the report and
// the in-order commits.  Host code only; the kernels are those of the other
// entry points.
//
// The schedule needs each step's commit counts before it can plan the next
// step.  The unmask's decision kernel writes them straight into host memory
// mapped for the device, and the host polls that memory: no copy is
// enqueued and the stream is not synchronised, so the next step starts as
// soon as the counts land.

#include <hip/hip_runtime.h>

#include <chrono>
#include <cstring>
#include <mutex>

#include "bc.h"
#include "pipeline_state.h"

namespace {

// Host memory for the commit counts, one buffer per device: mapped for the
// device and coherent, so the kernel's stores reach it without a copy.
// Allocated on first use and kept until the process ends; a decode holds
// its device's lock for its whole loop.
constexpr int kMaxDevices = 64;
struct CountsBuffer {
  std::mutex use;
  int32_t* host = nullptr;
  int32_t* dev = nullptr;
};
CountsBuffer g_counts[kMaxDevices];
std::mutex g_counts_init;

int counts_buffer(int device, CountsBuffer*& out) {
  if (device < 0 || device >= kMaxDevices) return BC_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> g(g_counts_init);
  CountsBuffer& b = g_counts[device];
  if (!b.host) {
    void* h = nullptr;
    if (hipHostMalloc(&h, BC_MAX_BLOCKS * sizeof(int32_t), hipHostMallocMapped | hipHostMallocCoherent) !=
        hipSuccess)
      return BC_ERR_HIP;
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, h, 0) != hipSuccess) {
      (void)hipHostFree(h);
      return BC_ERR_HIP;
    }
    b.host = static_cast<int32_t*>(h);
    b.dev = static_cast<int32_t*>(d);
  }
  out = &b;
  return BC_OK;
}

// Wait until the n counts (set to -1 before the step) have been written.
// Every few thousand reads the stream is asked whether it failed or has
// drained; a drained stream with counts still missing, or a minute without
// them, is reported as a runtime error rather than waited on forever.
int wait_counts(const volatile int32_t* c, int n, hipStream_t s) {
  const auto t0 = std::chrono::steady_clock::now();
  for (unsigned spin = 1;; ++spin) {
    bool ready = true;
    for (int j = 0; j < n && ready; ++j) ready = c[j] >= 0;
    if (ready) return BC_OK;
    if (spin % 4096 == 0) {
      const hipError_t e = hipStreamQuery(s);
      if (e == hipSuccess) {
        for (int j = 0; j < n; ++j)
          if (c[j] < 0) return BC_ERR_HIP;
        return BC_OK;
      }
      if (e != hipErrorNotReady) return BC_ERR_HIP;
      if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(60)) return BC_ERR_HIP;
    }
  }
}

}  // namespace

extern "C" int bc_pipeline_decode(bc_pipeline* p, const bc_kv_cache* cache, int32_t* cache_len,
                                  int32_t n_q_heads, int32_t vocab, float scale, float threshold,
                                  uint8_t* masked, int32_t* tokens, void* out, void* ws_attn,
                                  size_t ws_attn_bytes, void* ws_unmask, size_t ws_unmask_bytes,
                                  bc_step_inputs_fn inputs, bc_after_attn_fn after_attn, void* user,
                                  int32_t* trace, int32_t max_steps, int32_t* n_steps, void* stream) {
  if (!p || !cache || !cache_len || !masked || !tokens || !out || !inputs || !n_steps || max_steps < 0)
    return BC_ERR_ARG;
  if (cache->n_seq != 1) return BC_ERR_ARG;
  *n_steps = 0;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return BC_ERR_HIP;
  CountsBuffer* cb = nullptr;
  int rc = counts_buffer(device, cb);
  if (rc != BC_OK) return rc;
  std::lock_guard<std::mutex> hold(cb->use);

  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int W = p->window;
  const int stride = BC_PIPE_TRACE_INTS(W);
  int32_t active[BC_MAX_BLOCKS], local[BC_MAX_BLOCKS], mode[BC_MAX_BLOCKS], ndiv[BC_MAX_BLOCKS];
  int32_t off[BC_MAX_BLOCKS + 1], done[BC_MAX_BLOCKS], counts[BC_MAX_BLOCKS];
  int32_t row0 = 0;
  for (int step = 0;; ++step) {
    const int n = bc_pipeline_next(p, active, local, mode, ndiv, off, &row0);
    if (n < 0) return n;
    if (n == 0) break;
    if (trace && step >= max_steps) return BC_ERR_CAPACITY;

    bc_step_inputs in;
    std::memset(&in, 0, sizeof(in));
    if (inputs(user, step, n, active, local, &in) != 0) return BC_ERR_CALLBACK;

    const bc_active a{in.q, in.k, in.v, off, n, 1, off[n], n_q_heads};
    rc = bc_attn_step(cache, cache_len, nullptr, nullptr, &a, BC_MASK_BLOCK_BIDIR, scale, 0, out, ws_attn,
                      ws_attn_bytes, stream);
    if (rc != BC_OK) return rc;
    if (after_attn && after_attn(user, step, n, active, local, cache_len[0], out) != 0) return BC_ERR_CALLBACK;

    volatile int32_t* c = cb->host;
    for (int j = 0; j < n; ++j) c[j] = -1;
    rc = bc_unmask_select(in.logits, off[n], vocab, off, n, mode, ndiv, threshold, masked + row0, tokens + row0,
                          nullptr, cb->dev, ws_unmask, ws_unmask_bytes, stream);
    if (rc != BC_OK) return rc;
    rc = wait_counts(c, n, s);
    if (rc != BC_OK) return rc;
    for (int j = 0; j < n; ++j) counts[j] = c[j];

    const int nd = bc_pipeline_report(p, counts, done);
    if (nd < 0) return nd;
    for (int d = 0; d < nd; ++d) {   // completed blocks are active in the step that completes them
      const int j = done[d] - active[0];
      if (j < 0 || j >= n) return BC_ERR_ORDER;
      rc = bc_kv_commit(cache, cache_len, 0, cache_len[0], p->size[done[d]], in.blk_k[j], in.blk_v[j], stream);
      if (rc != BC_OK) return rc;
    }
    if (trace) {
      int32_t* r = trace + (size_t)step * stride;
      for (int k = 0; k < stride; ++k) r[k] = -1;
      r[0] = n;
      r[1] = nd;
      for (int j = 0; j < n; ++j) {
        r[2 + j] = active[j];
        r[2 + W + j] = mode[j];
        r[2 + 2 * W + j] = counts[j];
      }
      for (int d = 0; d < nd; ++d) r[2 + 3 * W + d] = done[d];
    }
    *n_steps = step + 1;
  }
  return BC_OK;
}
