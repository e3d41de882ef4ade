// Pipelined parallel decoding with the schedule on the device (Fast-dVLA
// reading notes, key design 4): the state machine of pipeline.hip run by a
// one-workgroup kernel after each step's unmask.  It takes the step's commit
// counts, appends the completed blocks to the cache in order, and writes the
// next step's plan (bc_dev_plan) into device memory.  The step's attention
// and unmask kernels read their rows, blocks, modes and cache length from
// that plan, so a step never waits for the host and runs of steps can be
// captured in one graph.
//
// Host side: bc_pipeline_dev_* (include/bc.h).  The attention and unmask
// arguments are prepared once, for the widest step (R rows, the cache's
// capacity); the plan then narrows them on the device.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include "bc_internal.h"

using namespace bc;

namespace {

enum : int { kWait = 0, kSemi = 1, kFull = 2 };
enum : int { kCommitted = 0, kSteps = 1, kLen = 2, kError = 3, kRow0 = 4, kScalars = 8 };
enum : int { kErrCount = 1, kErrTrace = 2, kErrInput = 3 };

struct SchedArgs {
  int* size;        // [nb] device state
  int* revealed;
  int* local;
  int* state;
  int* scal;        // kScalars ints: committed, steps, len, error, row0
  bc_dev_plan* plan;
  const int* n_commit;   // [window], written by the step's unmask
  int* trace;            // [max_steps][2 + 4 window]
  int* status;           // host-mapped: finished, steps, len, error
  const unsigned char* step_k;   // [Hkv][R][D] of the step
  const unsigned char* step_v;
  unsigned char* cache_k;        // sequence 0: [Hkv][cap][D]
  unsigned char* cache_v;
  int nb, window, n_div, max_steps, R, Hkv, row_bytes, cap, prefix;
  double add, act;
  int reset;
};

// The state of the blocks a step can touch, staged in LDS: blocks
// c0 .. c0 + kSpan - 1 (c0 the oldest uncommitted block when the kernel
// starts).  A step's blocks are at most `window` from c0, its commits at most
// `window` more, and the next plan at most `window` from the new oldest
// block, plus the first waiting block the transitions look at.
constexpr int kSpan = 2 * BC_MAX_BLOCKS + 2;
// With at most kAllBlocks blocks every block is staged, in the same round of
// loads as the scalars (no wait for the oldest uncommitted block's index).
constexpr int kAllBlocks = 512;
constexpr int kStaged = kAllBlocks > kSpan ? kAllBlocks : kSpan;
struct Staged {
  int scal[kScalars];
  int size[kStaged], revealed[kStaged], local[kStaged], state[kStaged];
  int n, blk_off[BC_MAX_BLOCKS + 1], active[BC_MAX_BLOCKS], mode[BC_MAX_BLOCKS], counts[BC_MAX_BLOCKS];
  int nd, len0, src[BC_MAX_BLOCKS], rows[BC_MAX_BLOCKS];
  bc_dev_plan next;
};

// The schedule's transitions and the next plan (one thread, on the staged
// state; block b is entry b - c0, c0 the first staged block), as
// bc_pipeline_next makes them: the
// oldest uncommitted block is fully active; walking forward while the
// predecessor is active, a waiting block joins as semi-active once its
// predecessor's completion ratio exceeds `add` (and fewer than `window`
// blocks are active), and a semi-active block turns fully active once the
// ratio exceeds `act`.
__device__ void plan_next(const SchedArgs& a, Staged& g, int c0) {
  bc_dev_plan& p = g.next;
  const int c = g.scal[kCommitted];
  p.row0 = g.scal[kRow0];
  p.len = g.scal[kLen];
  p.blk_off[0] = 0;
  if (c >= a.nb || g.scal[kError]) {
    p.n = p.rows = p.n_blk = 0;
    return;
  }
  const int end = min(a.nb, c0 + (a.nb <= kAllBlocks ? kAllBlocks : kSpan));
  g.state[c - c0] = kFull;
  int n_active = 0;
  for (int b = c; b < end && g.state[b - c0] != kWait; ++b) ++n_active;
  for (int b = c + 1; b < end; ++b) {
    if (g.state[b - 1 - c0] == kWait) break;   // blocks join in order
    const double r = (double)g.revealed[b - 1 - c0] / (double)g.size[b - 1 - c0];
    if (g.state[b - c0] == kWait && r > a.add && n_active < a.window) {
      g.state[b - c0] = kSemi;
      ++n_active;
    }
    if (g.state[b - c0] == kSemi && r > a.act) g.state[b - c0] = kFull;
  }
  int n = 0;
  for (int b = c; b < end && g.state[b - c0] != kWait; ++b, ++n) {
    p.active[n] = b;
    p.local_step[n] = g.local[b - c0];
    p.mode[n] = g.state[b - c0] == kFull ? BC_UNMASK_FULL : BC_UNMASK_SEMI;
    p.n_div[n] = g.state[b - c0] == kFull ? a.n_div : 1;
    p.blk_off[n + 1] = p.blk_off[n] + g.size[b - c0];
  }
  p.n = n;
  p.rows = p.blk_off[n];
  p.n_blk = n;
  if (p.rows < a.R) p.blk_off[++p.n_blk] = a.R;   // the idle rows: one more block, seen by no active row
}

// The report of the planned step (one thread, on the staged state): its
// counts checked and added, the blocks it completed (strictly in order), the
// trace record.
__device__ void report(const SchedArgs& a, Staged& g, int c0) {
  g.nd = 0;
  g.len0 = g.scal[kLen];
  const int n = g.n;
  if (n <= 0 || g.scal[kError]) return;
  bool ok = true;
  for (int j = 0; j < n; ++j) {
    const int e = g.active[j] - c0, k = g.counts[j];
    ok = ok && k >= 0 && k <= g.size[e] - g.revealed[e];
  }
  const int step = g.scal[kSteps];
  if (!ok) {
    g.scal[kError] = kErrCount;
    return;
  }
  if (step >= a.max_steps) {
    g.scal[kError] = kErrTrace;
    return;
  }
  for (int j = 0; j < n; ++j) {
    const int e = g.active[j] - c0;
    g.revealed[e] += g.counts[j];
    g.local[e] += 1;
  }
  int c = g.scal[kCommitted], nd = 0;
  // completed blocks are the oldest active ones: the plan's first blocks
  while (c < a.nb && c - g.active[0] < n && g.state[c - c0] != kWait && g.revealed[c - c0] == g.size[c - c0]) {
    g.src[nd] = g.blk_off[c - g.active[0]];   // the block's rows in the step buffers
    g.rows[nd] = g.size[c - c0];
    g.scal[kLen] += g.size[c - c0];
    g.scal[kRow0] += g.size[c - c0];
    ++nd;
    ++c;
  }
  int* r = a.trace + (long long)step * (2 + 4 * a.window);
  for (int i = 0; i < 2 + 4 * a.window; ++i) r[i] = -1;
  r[0] = n;
  r[1] = nd;
  for (int j = 0; j < n; ++j) {
    r[2 + j] = g.active[j];
    r[2 + a.window + j] = g.mode[j];
    r[2 + 2 * a.window + j] = g.counts[j];
  }
  for (int d = 0; d < nd; ++d) r[2 + 3 * a.window + d] = g.scal[kCommitted] + d;
  g.scal[kCommitted] = c;
  g.scal[kSteps] = step + 1;
  g.nd = nd;
}

__device__ void write_status(const SchedArgs& a, const Staged& g) {
  a.status[0] = (g.scal[kCommitted] >= a.nb || g.scal[kError]) ? 1 : 0;
  a.status[1] = g.scal[kSteps];
  a.status[2] = g.scal[kLen];
  a.status[3] = g.scal[kError];
}

// One workgroup.  The state it needs is staged in LDS in two parallel
// rounds of loads (the scalars, the plan and the counts; then the blocks
// from the oldest uncommitted one), thread 0 runs the schedule there, and
// the results go back in parallel.  reset: initial state and the first
// plan.  Otherwise: the report of the planned step, the commits of the
// blocks it completed (all threads copy their K/V rows), the next plan.
__global__ __launch_bounds__(256) void sched_kernel(const SchedArgs a) {
  __shared__ Staged g;
  const int t = threadIdx.x;
  if (a.reset) {
    for (int b = t; b < a.nb; b += blockDim.x) {
      a.revealed[b] = 0;
      a.local[b] = 0;
      a.state[b] = kWait;
    }
    if (t < kScalars) g.scal[t] = t == kLen ? a.prefix : 0;
    g.n = 0;
  } else {
    if (t < kScalars) g.scal[t] = a.scal[t];
    const bc_dev_plan* p = a.plan;
    if (t == 0) g.n = p->n;
    if (t < BC_MAX_BLOCKS) {
      g.active[t] = p->active[t];
      g.mode[t] = p->mode[t];
      g.counts[t] = a.n_commit[t];
    }
    if (t <= BC_MAX_BLOCKS) g.blk_off[t] = p->blk_off[t];
  }
  // the blocks: all of them with the scalars, or, past kAllBlocks blocks,
  // kSpan from the oldest uncommitted one once its index has arrived
  const bool all = a.nb <= kAllBlocks;
  auto stage_blocks = [&](int first, int count) {
    for (int e = t; e < count; e += blockDim.x) {
      const int b = first + e;
      if (b < a.nb) {
        g.size[e] = a.size[b];
        g.revealed[e] = a.reset ? 0 : a.revealed[b];
        g.local[e] = a.reset ? 0 : a.local[b];
        g.state[e] = a.reset ? kWait : a.state[b];
      }
    }
  };
  if (all) stage_blocks(0, a.nb);
  __syncthreads();
  const int c0 = all ? 0 : g.scal[kCommitted];
  const int span = all ? a.nb : kSpan;
  if (!all) {
    stage_blocks(c0, kSpan);
    __syncthreads();
  }
  if (t == 0) {
    if (!a.reset) report(a, g, c0);
    else g.nd = 0, g.len0 = g.scal[kLen];
    plan_next(a, g, c0);
  }
  __syncthreads();
  // write-back: the staged blocks' state, the scalars, the next plan
  for (int e = t; e < span; e += blockDim.x) {
    const int b = c0 + e;
    if (b < a.nb) {
      a.revealed[b] = g.revealed[e];
      a.local[b] = g.local[e];
      a.state[b] = g.state[e];
    }
  }
  if (t < kScalars) a.scal[t] = g.scal[t];
  {
    const int* src = reinterpret_cast<const int*>(&g.next);
    int* dst = reinterpret_cast<int*>(a.plan);
    for (int i = t; i < (int)(sizeof(bc_dev_plan) / sizeof(int)); i += blockDim.x) dst[i] = src[i];
  }
  if (t == 0) write_status(a, g);
  // the commits: block d's rows [src, src + rows) of every head, to cache
  // rows starting at the length before it (16-byte units)
  const int units_per_row = a.row_bytes / 16;
  int dst = g.len0;
  for (int d = 0; d < g.nd; ++d) {
    const int n_units = a.Hkv * g.rows[d] * units_per_row;
    for (int u = t; u < n_units; u += blockDim.x) {
      const int h = u / (g.rows[d] * units_per_row);
      const int rem = u - h * g.rows[d] * units_per_row;
      const int row = rem / units_per_row, part = rem - row * units_per_row;
      const long long src = ((long long)h * a.R + g.src[d] + row) * a.row_bytes + part * 16;
      const long long out = ((long long)h * a.cap + dst + row) * a.row_bytes + part * 16;
      *reinterpret_cast<uint4*>(a.cache_k + out) = *reinterpret_cast<const uint4*>(a.step_k + src);
      *reinterpret_cast<uint4*>(a.cache_v + out) = *reinterpret_cast<const uint4*>(a.step_v + src);
    }
    dst += g.rows[d];
  }
}

struct ReplayArgs {
  const bc_step_block* table;
  int max_local;
  const bc_dev_plan* plan;
  const int* size;
  int* scal;
  unsigned char *q, *k, *v, *logits;   // step buffers
  int R, q_row_bytes, kv_row_bytes, Hkv, logit_row_bytes;
};

// Copy of the planned blocks' recorded rows into the step buffers: block j
// of the plan is workgroup row blockIdx.y == j; the x workgroups share its
// bytes in 16-byte units.
__global__ __launch_bounds__(256) void replay_kernel(const ReplayArgs a) {
  const bc_dev_plan* p = a.plan;
  const int j = blockIdx.y;
  if (j >= p->n) return;
  const int b = p->active[j], s = p->local_step[j];
  const bc_step_block* e = (s < a.max_local) ? &a.table[(long long)b * a.max_local + s] : nullptr;
  if (!e || !e->q || !e->k || !e->v || !e->logits) {
    if (threadIdx.x == 0 && blockIdx.x == 0) a.scal[kError] = kErrInput;
    return;
  }
  const int rows = a.size[b], off = p->blk_off[j];
  const long long nq = (long long)rows * a.q_row_bytes / 16, nl = (long long)rows * a.logit_row_bytes / 16;
  const long long nkv_head = (long long)rows * a.kv_row_bytes / 16, nkv = nkv_head * a.Hkv;
  const long long total = nq + 2 * nkv + nl;
  const unsigned char* eq = static_cast<const unsigned char*>(e->q);
  const unsigned char* ek = static_cast<const unsigned char*>(e->k);
  const unsigned char* ev = static_cast<const unsigned char*>(e->v);
  const unsigned char* el = reinterpret_cast<const unsigned char*>(e->logits);
  for (long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x; u < total;
       u += (long long)gridDim.x * blockDim.x) {
    const unsigned char* src;
    unsigned char* dst;
    if (u < nq) {
      src = eq + u * 16;
      dst = a.q + (long long)off * a.q_row_bytes + u * 16;
    } else if (u < nq + 2 * nkv) {
      long long w = u - nq;
      const bool is_v = w >= nkv;
      if (is_v) w -= nkv;
      const long long h = w / nkv_head, r = w - h * nkv_head;
      src = (is_v ? ev : ek) + w * 16;
      dst = (is_v ? a.v : a.k) + (h * a.R + off) * a.kv_row_bytes + r * 16;
    } else {
      const long long w = u - nq - 2 * nkv;
      src = el + w * 16;
      dst = a.logits + (long long)off * a.logit_row_bytes + w * 16;
    }
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
}

int elem_size(int dtype) { return dtype == BC_BF16 ? 2 : 4; }

}  // namespace

struct bc_pipeline_dev {
  int device = 0;
  std::vector<int> sizes;
  int nb = 0, window = 1, R = 0, max_steps = 0, Hq = 0, Hkv = 0, D = 0, V = 0, dtype = 0;
  bc_kv_cache cache{};
  void* mem = nullptr;           // device: state, plan, counts, trace, workspaces
  int32_t* status_host = nullptr;
  int32_t* status_dev = nullptr;
  SchedArgs sched{};
  AttnArgs attn{};
  UnmaskArgs unmask{};
  ReplayArgs replay{};
};

extern "C" {

int bc_pipeline_dev_create(const int32_t* block_sizes, int32_t n_blocks, int32_t window, double add, double act,
                           int32_t n_div, const bc_kv_cache* cache, int32_t prefix_len, int32_t n_q_heads,
                           int32_t vocab, float scale, float threshold, uint8_t* masked, int32_t* tokens, void* q,
                           void* k, void* v, float* logits, void* out, int32_t max_steps, bc_pipeline_dev** dev) {
  if (!dev) return BC_ERR_ARG;
  *dev = nullptr;
  if (!block_sizes || n_blocks < 1 || n_blocks > 4096 || window < 1 || window > BC_MAX_BLOCKS || n_div < 1 ||
      !std::isfinite(add) || !std::isfinite(act) || !cache || cache->n_seq != 1 || !cache->k || !cache->v ||
      !masked || !tokens || !q || !k || !v || !logits || !out || max_steps < 1 || vocab < 1)
    return BC_ERR_ARG;
  long long total = 0;
  for (int b = 0; b < n_blocks; ++b) {
    if (block_sizes[b] < 1) return BC_ERR_ARG;
    total += block_sizes[b];
  }
  if (prefix_len < 0 || prefix_len + total > cache->capacity) return BC_ERR_ARG;
  if (vocab % 4 != 0) return BC_ERR_UNSUPPORTED;   // the replay copies logit rows in 16-byte units
  // R: the widest step, the largest sum of `window` consecutive blocks
  int R = 0, widest = 0;
  for (int b = 0; b < n_blocks; ++b) {
    int r = 0;
    for (int j = b; j < n_blocks && j < b + window; ++j) r += block_sizes[j];
    if (r > R) R = r, widest = b;
  }
  // the widest step's arguments, validated with that step's blocks (the
  // plan replaces the offsets, modes and n on the device)
  std::vector<int32_t> off = {0};
  for (int j = widest; j < n_blocks && j < widest + window; ++j) off.push_back(off.back() + block_sizes[j]);
  const int n_w = (int)off.size() - 1;
  std::vector<int32_t> mode(n_w, BC_UNMASK_FULL), div(n_w, 1);
  const bc_active a{q, k, v, off.data(), n_w, 1, R, n_q_heads};
  const size_t ws_attn = bc_attn_workspace_bytes(cache, nullptr, &a, 0);
  const size_t ws_unmask = bc_unmask_workspace_bytes(R, vocab);
  if (ws_attn == 0 || ws_unmask == 0) return BC_ERR_UNSUPPORTED;

  bc_pipeline_dev* d = new (std::nothrow) bc_pipeline_dev;
  if (!d) return BC_ERR_ARG;
  d->sizes.assign(block_sizes, block_sizes + n_blocks);
  d->nb = n_blocks;
  d->window = window;
  d->R = R;
  d->max_steps = max_steps;
  d->Hq = n_q_heads;
  d->Hkv = cache->n_kv_heads;
  d->D = cache->head_dim;
  d->V = vocab;
  d->dtype = cache->dtype;
  d->cache = *cache;
  if (hipGetDevice(&d->device) != hipSuccess) {
    delete d;
    return BC_ERR_HIP;
  }

  // one device allocation, carved in 256-byte aligned pieces
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t b_state = al(4 * sizeof(int) * n_blocks), b_scal = al(kScalars * sizeof(int));
  const size_t b_plan = al(sizeof(bc_dev_plan)), b_counts = al(BC_MAX_BLOCKS * sizeof(int));
  const size_t b_trace = al((size_t)max_steps * (2 + 4 * window) * sizeof(int));
  const size_t bytes = b_state + b_scal + b_plan + b_counts + b_trace + al(ws_attn) + al(ws_unmask);
  if (hipMalloc(&d->mem, bytes) != hipSuccess) {
    delete d;
    return BC_ERR_HIP;
  }
  void* h = nullptr;
  if (hipHostMalloc(&h, 4 * sizeof(int32_t), hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess) {
    (void)hipFree(d->mem);
    delete d;
    return BC_ERR_HIP;
  }
  d->status_host = static_cast<int32_t*>(h);
  std::memset(d->status_host, 0, 4 * sizeof(int32_t));
  void* hd = nullptr;
  if (hipHostGetDevicePointer(&hd, h, 0) != hipSuccess) {
    bc_pipeline_dev_destroy(d);
    return BC_ERR_HIP;
  }
  d->status_dev = static_cast<int32_t*>(hd);
  char* m = static_cast<char*>(d->mem);
  int* state = reinterpret_cast<int*>(m);
  int* scal = reinterpret_cast<int*>(m + b_state);
  bc_dev_plan* plan = reinterpret_cast<bc_dev_plan*>(m + b_state + b_scal);
  int* counts = reinterpret_cast<int*>(m + b_state + b_scal + b_plan);
  int* trace = reinterpret_cast<int*>(m + b_state + b_scal + b_plan + b_counts);
  void* wa = m + b_state + b_scal + b_plan + b_counts + b_trace;
  void* wu = static_cast<char*>(wa) + al(ws_attn);
  // the block sizes never change: copied once (blocking; the rest of the
  // state is set by the reset kernel)
  if (hipMemcpy(state, block_sizes, sizeof(int) * n_blocks, hipMemcpyHostToDevice) != hipSuccess) {
    bc_pipeline_dev_destroy(d);
    return BC_ERR_HIP;
  }

  const int32_t len_max = cache->capacity;
  int st = prepare_attn_args(cache, &len_max, &a, scale, out, wa, ws_attn, &d->attn);
  if (st == BC_OK)
    st = prepare_unmask_args(logits, R, vocab, off.data(), n_w, mode.data(), div.data(), threshold, masked, tokens,
                             counts, wu, ws_unmask, &d->unmask);
  if (st != BC_OK) {
    bc_pipeline_dev_destroy(d);
    return st;
  }
  d->attn.dyn = plan;
  d->unmask.dyn = plan;
  d->unmask.n_blk = window;   // one decision workgroup per possible active block

  SchedArgs& s = d->sched;
  s.size = state;
  s.revealed = state + n_blocks;
  s.local = state + 2 * n_blocks;
  s.state = state + 3 * n_blocks;
  s.scal = scal;
  s.plan = plan;
  s.n_commit = counts;
  s.trace = trace;
  s.status = d->status_dev;
  s.step_k = static_cast<const unsigned char*>(k);
  s.step_v = static_cast<const unsigned char*>(v);
  s.cache_k = static_cast<unsigned char*>(cache->k);
  s.cache_v = static_cast<unsigned char*>(cache->v);
  s.nb = n_blocks;
  s.window = window;
  s.n_div = n_div;
  s.max_steps = max_steps;
  s.R = R;
  s.Hkv = cache->n_kv_heads;
  s.row_bytes = cache->head_dim * elem_size(cache->dtype);
  s.cap = cache->capacity;
  s.prefix = prefix_len;
  s.add = add;
  s.act = act;

  ReplayArgs& r = d->replay;
  r.plan = plan;
  r.size = state;
  r.scal = scal;
  r.q = static_cast<unsigned char*>(q);
  r.k = static_cast<unsigned char*>(k);
  r.v = static_cast<unsigned char*>(v);
  r.logits = reinterpret_cast<unsigned char*>(logits);
  r.R = R;
  r.q_row_bytes = n_q_heads * cache->head_dim * elem_size(cache->dtype);
  r.kv_row_bytes = cache->head_dim * elem_size(cache->dtype);
  r.Hkv = cache->n_kv_heads;
  r.logit_row_bytes = vocab * (int)sizeof(float);
  *dev = d;
  return BC_OK;
}

void bc_pipeline_dev_destroy(bc_pipeline_dev* d) {
  if (!d) return;
  (void)hipDeviceSynchronize();
  if (d->mem) (void)hipFree(d->mem);
  if (d->status_host) (void)hipHostFree(d->status_host);
  delete d;
}

int bc_pipeline_dev_rows(const bc_pipeline_dev* d) { return d ? d->R : BC_ERR_ARG; }

const bc_dev_plan* bc_pipeline_dev_plan(const bc_pipeline_dev* d) { return d ? d->sched.plan : nullptr; }

int bc_pipeline_dev_reset(bc_pipeline_dev* d, void* stream) {
  if (!d) return BC_ERR_ARG;
  SchedArgs a = d->sched;
  a.reset = 1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(256), 0, static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? BC_OK : BC_ERR_HIP;
}

int bc_pipeline_dev_step(bc_pipeline_dev* d, void* stream) {
  if (!d) return BC_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (launch_attn_partial(d->attn, d->dtype, s) != hipSuccess) return BC_ERR_HIP;
  if (launch_attn_combine(d->attn, d->dtype, s) != hipSuccess) return BC_ERR_HIP;
  if (launch_scan(d->unmask.logits, d->R, d->V, d->unmask.masked, true, const_cast<ScanPartial*>(d->unmask.part), s,
                  d->unmask.dyn) != hipSuccess)
    return BC_ERR_HIP;
  if (launch_unmask_decide(d->unmask, s) != hipSuccess) return BC_ERR_HIP;
  SchedArgs a = d->sched;
  a.reset = 0;
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? BC_OK : BC_ERR_HIP;
}

int bc_pipeline_dev_replay(bc_pipeline_dev* d, const bc_step_block* table, int32_t max_local, void* stream) {
  if (!d || !table || max_local < 1) return BC_ERR_ARG;
  ReplayArgs a = d->replay;
  a.table = table;
  a.max_local = max_local;
  (void)hipGetLastError();
  hipLaunchKernelGGL(replay_kernel, dim3(128, d->window), dim3(256), 0, static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? BC_OK : BC_ERR_HIP;
}

int bc_pipeline_dev_status(const bc_pipeline_dev* d, int32_t* finished, int32_t* n_steps, int32_t* cache_len,
                           int32_t* error) {
  if (!d) return BC_ERR_ARG;
  const volatile int32_t* st = d->status_host;
  if (finished) *finished = st[0];
  if (n_steps) *n_steps = st[1];
  if (cache_len) *cache_len = st[2];
  if (error) *error = st[3];
  return BC_OK;
}

int bc_pipeline_dev_trace(const bc_pipeline_dev* d, int32_t* trace, int32_t max_steps) {
  if (!d || !trace || max_steps < 0) return BC_ERR_ARG;
  if (hipDeviceSynchronize() != hipSuccess) return BC_ERR_HIP;   // the status and trace are final
  const int n = std::min(max_steps, (int)static_cast<const volatile int32_t*>(d->status_host)[1]);
  if (n <= 0) return 0;
  if (hipMemcpy(trace, d->sched.trace, sizeof(int32_t) * n * (2 + 4 * d->window), hipMemcpyDeviceToHost) !=
      hipSuccess)
    return BC_ERR_HIP;
  return n;
}

int bc_pipeline_dev_read_plan(const bc_pipeline_dev* d, bc_dev_plan* plan) {
  if (!d || !plan) return BC_ERR_ARG;
  if (hipDeviceSynchronize() != hipSuccess) return BC_ERR_HIP;
  return hipMemcpy(plan, d->sched.plan, sizeof(bc_dev_plan), hipMemcpyDeviceToHost) == hipSuccess ? BC_OK
                                                                                                : BC_ERR_HIP;
}

}  // extern "C"
