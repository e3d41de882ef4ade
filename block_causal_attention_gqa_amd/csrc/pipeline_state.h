// State of the pipelined parallel decoding schedule (bc_pipeline_*), shared
// by the state machine (pipeline.hip) and the native decode loop
// (pipeline_run.hip).  Host memory only.
#pragma once

#include <vector>

struct bc_pipeline {
  std::vector<int> size, revealed, local, state;
  int committed = 0, window = 1, n_div = 1;
  double add = 0.0, act = 0.0;
  std::vector<int> plan;   // the planned step's blocks (empty: no plan)
};
