// Pipelined parallel decoding schedule: the host-side state machine behind
// bc_pipeline_* (Fast-dVLA reading notes, key design 4).  No GPU code.
//
// Per block: its size, rows revealed so far, steps it has been active, and
// its state -- waiting, semi-active (threshold-only commits) or fully
// active (threshold plus the ceil(remaining / n) fallback).  Before each
// step the states move: the oldest uncommitted block is fully active; walking
// forward while the predecessor is active, a waiting block joins as
// semi-active once its predecessor's completion ratio exceeds `add` (and
// fewer than `window` blocks are active), and a semi-active block becomes
// fully active once that ratio exceeds `act`.  "Exceeds" is strict, as for
// the confidence threshold: the notes use the one word for all three.
// After the step the reported counts are added and completed blocks are
// committed strictly in order.

#include <cmath>
#include <new>
#include <vector>

#include "bc.h"
#include "pipeline_state.h"

namespace {

enum : int { kWait = 0, kSemi = 1, kFull = 2 };

// revealed / size, rounded once (double): a ratio equal to a threshold
// stays equal to it and so does not exceed it
double ratio(const bc_pipeline& p, int b) { return (double)p.revealed[b] / (double)p.size[b]; }

void transitions(bc_pipeline& p) {
  const int n = (int)p.size.size();
  p.state[p.committed] = kFull;
  int n_active = 0;
  for (int b = p.committed; b < n; ++b) n_active += p.state[b] != kWait;
  for (int b = p.committed + 1; b < n; ++b) {
    if (p.state[b - 1] == kWait) break;   // blocks join in order
    const double r = ratio(p, b - 1);
    if (p.state[b] == kWait && r > p.add && n_active < p.window) {
      p.state[b] = kSemi;
      ++n_active;
    }
    if (p.state[b] == kSemi && r > p.act) p.state[b] = kFull;
  }
}

}  // namespace

extern "C" {

int bc_pipeline_create(const int32_t* block_sizes, int32_t n_blocks, int32_t window, double add, double act,
                       int32_t n_div, bc_pipeline** out) {
  if (!out) return BC_ERR_ARG;
  *out = nullptr;
  if (!block_sizes || n_blocks < 1 || n_blocks > 4096 || window < 1 || window > BC_MAX_BLOCKS || n_div < 1 ||
      !std::isfinite(add) || !std::isfinite(act))
    return BC_ERR_ARG;
  for (int b = 0; b < n_blocks; ++b)
    if (block_sizes[b] < 1) return BC_ERR_ARG;
  bc_pipeline* p = new (std::nothrow) bc_pipeline;
  if (!p) return BC_ERR_ARG;
  p->size.assign(block_sizes, block_sizes + n_blocks);
  p->revealed.assign(n_blocks, 0);
  p->local.assign(n_blocks, 0);
  p->state.assign(n_blocks, kWait);
  p->window = window;
  p->n_div = n_div;
  p->add = add;
  p->act = act;
  *out = p;
  return BC_OK;
}

void bc_pipeline_destroy(bc_pipeline* p) { delete p; }

int bc_pipeline_next(bc_pipeline* p, int32_t* active, int32_t* local_step, int32_t* mode, int32_t* n_div,
                     int32_t* blk_off, int32_t* row0) {
  if (!p || !active || !local_step || !mode || !n_div || !blk_off || !row0) return BC_ERR_ARG;
  const int n = (int)p->size.size();
  if (p->committed == n) {
    p->plan.clear();
    return 0;
  }
  if (p->plan.empty()) {
    transitions(*p);
    for (int b = p->committed; b < n && p->state[b] != kWait; ++b) p->plan.push_back(b);
  }
  int r = 0;
  for (int b = 0; b < p->plan.front(); ++b) r += p->size[b];
  *row0 = r;
  blk_off[0] = 0;
  for (int j = 0; j < (int)p->plan.size(); ++j) {
    const int b = p->plan[j];
    active[j] = b;
    local_step[j] = p->local[b];
    mode[j] = p->state[b] == kFull ? BC_UNMASK_FULL : BC_UNMASK_SEMI;
    n_div[j] = p->state[b] == kFull ? p->n_div : 1;
    blk_off[j + 1] = blk_off[j] + p->size[b];
  }
  return (int)p->plan.size();
}

int bc_pipeline_report(bc_pipeline* p, const int32_t* n_commit, int32_t* done) {
  if (!p || !n_commit || !done) return BC_ERR_ARG;
  if (p->plan.empty()) return BC_ERR_ORDER;
  for (int j = 0; j < (int)p->plan.size(); ++j) {
    const int b = p->plan[j];
    if (n_commit[j] < 0 || n_commit[j] > p->size[b] - p->revealed[b]) return BC_ERR_ARG;
  }
  for (int j = 0; j < (int)p->plan.size(); ++j) {
    const int b = p->plan[j];
    p->revealed[b] += n_commit[j];
    p->local[b] += 1;
  }
  int k = 0;
  const int n = (int)p->size.size();
  while (p->committed < n && p->state[p->committed] != kWait &&
         p->revealed[p->committed] == p->size[p->committed])
    done[k++] = p->committed++;
  p->plan.clear();
  return k;
}

}  // extern "C"
