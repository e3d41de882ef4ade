// Vocabulary-wide row reductions and the decisions built on them.
//
//   unmask (Fast-dVLA notes, key design 4; Fast-dDrive method summary 3.1):
//     per still-masked row: max, lowest argmax and sum_v exp(l_v - max),
//     confidence = 1 / sum; then per block the threshold set A, the commit
//     count k (SEMI: |A|; FULL: min(|E|, max(|A|, ceil(|E| / n)))) and the
//     top-k rows by (confidence desc, row asc).
//   verify (Fast-dDrive method summary 3.2, Scaffold Speculative decoding):
//     per row the lowest argmax, then the first row from `first` whose draft
//     disagrees (scaffold rows pass) -> accept length and bonus token.  The
//     sampled variant (sec. 3.3, trajectory-only sampling) takes the argmax
//     of l / T + g with caller-supplied Gumbel noise g (Gumbel-max: a draw
//     from softmax(l / T)).
//
// Two kernels per call.  The scan is one pass over HBM: a (chunk, row) grid
// where each workgroup reads 4096 logits with 16-byte loads (4 per lane,
// all in flight before any arithmetic), reduces max / argmax / exp-sum inside
// the wave and across the 4 waves, and leaves one 16-byte partial.  Rows that
// need no scan (already revealed, or outside the verified range) skip the
// reads.  The decision kernel runs one workgroup per block (or sequence): it
// merges each row's chunk partials with 8 lanes per row, one round of loads,
// and decides.  The kernel boundary is the only synchronisation: no atomics,
// no counters, and the workspace needs no initialisation.
//
// Exact decisions.  Float32 confidences carry a relative error far below
// 2^-12.  A decision whose float32 margin -- to the threshold, or between the
// two sides of the ranking cut -- is inside that band is retaken on
// confidences recomputed in float64 by re-reading the row, so decisions
// follow the float64 confidences.

#include <climits>

#include "bc_internal.h"

namespace bc {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;
constexpr double kBand = 1.0 / 4096.0;   // relative float32 decision band

struct Acc { float m; int a; float s; };

__device__ inline Acc merge(Acc x, Acc y) {
  Acc r;
  r.m = fmaxf(x.m, y.m);
  r.a = (y.m > x.m || (y.m == x.m && y.a < x.a)) ? y.a : x.a;
  const float sx = x.m == kNegInf ? 0.f : x.s * __builtin_amdgcn_exp2f((x.m - r.m) * kLog2e);
  const float sy = y.m == kNegInf ? 0.f : y.s * __builtin_amdgcn_exp2f((y.m - r.m) * kLog2e);
  r.s = sx + sy;
  return r;
}

// Lane exchanges for the butterfly merges, all in VALU (no LDS round trip):
// DPP quad_perm [1,0,3,2] and [2,3,0,1] pair lanes 1 and 2 apart; once each
// quad (half row) holds one value, row_half_mirror (row_mirror) pairs it with
// the neighbouring quad (half row); v_permlane16_swap / v_permlane32_swap
// with both operands x return the two halves of each 16 (32) lane pair.
template <int kStep>
__device__ inline uint32_t lane_xchg(uint32_t x) {
  if constexpr (kStep == 0) return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);
  else if constexpr (kStep == 1) return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);
  else if constexpr (kStep == 2) return __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);
  else if constexpr (kStep == 3) return __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false);
  else {
    // the other half of the pair: swap returns (lower half, upper half) in
    // every lane, so the partner is whichever of the two is not this lane's
    const auto p = kStep == 4 ? __builtin_amdgcn_permlane16_swap(x, x, false, false)
                              : __builtin_amdgcn_permlane32_swap(x, x, false, false);
    const int bit = kStep == 4 ? 16 : 32;
    return (threadIdx.x & bit) ? (uint32_t)p[0] : (uint32_t)p[1];
  }
}

// Butterfly over aligned groups of kWidth lanes (8 or 64) on 32-bit values;
// `op` is commutative, so every lane of a group ends with the same bits.
template <int kWidth, typename Op>
__device__ inline uint32_t lanes_allreduce(uint32_t x, Op op) {
  static_assert(kWidth == 8 || kWidth == 64, "group width");
  x = op(x, lane_xchg<0>(x));
  x = op(x, lane_xchg<1>(x));
  x = op(x, lane_xchg<2>(x));
  if constexpr (kWidth == 64) {
    x = op(x, lane_xchg<3>(x));
    x = op(x, lane_xchg<4>(x));
    x = op(x, lane_xchg<5>(x));
  }
  return x;
}

template <int kWidth>
__device__ inline float lanes_max(float x) {
  return __builtin_bit_cast(float, lanes_allreduce<kWidth>(__builtin_bit_cast(uint32_t, x), [](uint32_t p, uint32_t q) {
    return __builtin_bit_cast(uint32_t, fmaxf(__builtin_bit_cast(float, p), __builtin_bit_cast(float, q)));
  }));
}

template <int kWidth>
__device__ inline float lanes_sum(float x) {
  return __builtin_bit_cast(float, lanes_allreduce<kWidth>(__builtin_bit_cast(uint32_t, x), [](uint32_t p, uint32_t q) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, p) + __builtin_bit_cast(float, q));
  }));
}

template <int kWidth>
__device__ inline int lanes_min(int x) {
  return (int)lanes_allreduce<kWidth>((uint32_t)x, [](uint32_t p, uint32_t q) { return (uint32_t)min((int)p, (int)q); });
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Logits (and noise) are read once: non-temporal loads stream them past L2
// and the MALL instead of evicting what the other calls of a step reuse
// (the K/V cache, the split partials).  Measured: the bs1 scan 5.25 -> 4.73
// us and the section decode +5%; the N = 64 verify 159 -> 146 us.
__device__ inline float4 stream_load4(const float* p) {
  const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return float4{t[0], t[1], t[2], t[3]};
}

// One (chunk, row) partial: max, lowest argmax and (kSum) exp-sum of
// logits[row][chunk * kScanChunk ...], written by thread 0.
// With kNoise the value scanned is l * inv_t + g (g from noisep at the same
// index): one float32 multiply and one float32 add, each rounded, never
// contracted into an FMA, so a float32 reference reproduces every value.
template <bool kSum, bool kVec, bool kNoise = false>
__device__ void scan_chunk(const float* __restrict__ rowp, int vocab, int chunk, ScanPartial* out,
                           Acc* red, const float* __restrict__ noisep = nullptr, float inv_t = 1.f) {
  const int tid = threadIdx.x;
  const int c0 = chunk * kScanChunk;
  const int c1 = min(vocab, c0 + kScanChunk);
  constexpr int NV = kScanVecPerThread * 4;
  float v[NV];
  if constexpr (kVec) {
#pragma unroll
    for (int it = 0; it < kScanVecPerThread; ++it) {
      const int idx = c0 + 4 * (tid + kScanThreads * it);
      float4 x = {kNegInf, kNegInf, kNegInf, kNegInf};
      if (idx < c1) {
        x = stream_load4(rowp + idx);
        if constexpr (kNoise) {
          const float4 g = stream_load4(noisep + idx);
          x = float4{__fadd_rn(__fmul_rn(x.x, inv_t), g.x), __fadd_rn(__fmul_rn(x.y, inv_t), g.y),
                     __fadd_rn(__fmul_rn(x.z, inv_t), g.z), __fadd_rn(__fmul_rn(x.w, inv_t), g.w)};
        }
      }
      v[4 * it] = x.x; v[4 * it + 1] = x.y; v[4 * it + 2] = x.z; v[4 * it + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const int idx = c0 + tid + kScanThreads * e;
      float x = kNegInf;
      if (idx < c1) {
        x = __builtin_nontemporal_load(rowp + idx);
        if constexpr (kNoise) x = __fadd_rn(__fmul_rn(x, inv_t), __builtin_nontemporal_load(noisep + idx));
      }
      v[e] = x;
    }
  }
  // Max first: the chunk max M over the lanes (butterfly) and the waves (one
  // LDS slot each); then every lane takes its lowest index holding M and its
  // sum of exp(l - M), and two more butterflies finish them.  No partial
  // result is ever rescaled, so the exponentials are the 16 per lane.
  auto index_of = [&](int e) {
    return kVec ? c0 + 4 * (tid + kScanThreads * (e / 4)) + (e & 3) : c0 + tid + kScanThreads * e;
  };
  const int w = tid >> 6;
  float m = v[0];
#pragma unroll
  for (int e = 1; e < NV; ++e) m = fmaxf(m, v[e]);
  m = lanes_max<64>(m);
  if ((tid & 63) == 0) red[w].m = m;
  __syncthreads();
  float M = red[0].m;
#pragma unroll
  for (int k = 1; k < kScanThreads / 64; ++k) M = fmaxf(M, red[k].m);
  int a = INT_MAX;
#pragma unroll
  for (int e = NV - 1; e >= 0; --e) a = v[e] == M ? index_of(e) : a;   // indices rise with e
  a = lanes_min<64>(a);
  float sum = 0.f;
  if constexpr (kSum) {
    if (M != kNegInf) {
#pragma unroll
      for (int e = 0; e < NV; ++e) sum += __builtin_amdgcn_exp2f((v[e] - M) * kLog2e);
    }
    sum = lanes_sum<64>(sum);
  }
  if ((tid & 63) == 0) {   // other fields than the maxima the slower waves may still read
    red[w].a = a;
    red[w].s = sum;
  }
  __syncthreads();
  if (tid == 0) {
    int at = red[0].a;
    float st = red[0].s;
#pragma unroll
    for (int k = 1; k < kScanThreads / 64; ++k) {
      at = min(at, red[k].a);
      st += red[k].s;
    }
    *out = ScanPartial{M, at, kSum ? st : 0.f, 0};
  }
}

// mode 0: rows with row_mask[row] != 0 (all rows when row_mask is null);
// mode 1: verify, row (s, i) with first[s] <= i <= min(m, n_lrows - 1).
template <int kMode, bool kSum, bool kVec, bool kNoise = false, bool kDyn = false>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(const float* __restrict__ logits, int vocab,
                                                             int n_chunks, ScanPartial* __restrict__ part,
                                                             const uint8_t* __restrict__ row_mask,
                                                             const int* __restrict__ first, int n_lrows,
                                                             int m, const float* __restrict__ noise = nullptr,
                                                             float inv_t = 1.f,
                                                             const DevPlan* __restrict__ dyn = nullptr) {
  __shared__ Acc red[kScanThreads / 64];
  const int chunk = blockIdx.x, row = blockIdx.y;
  if constexpr (kMode == 0) {
    if constexpr (kDyn) {   // device-resident plan: its rows only, flags at its row0
      if (row >= __builtin_amdgcn_readfirstlane(dyn->rows) ||
          !row_mask[__builtin_amdgcn_readfirstlane(dyn->row0) + row])
        return;
    } else if (row_mask && !row_mask[row]) {
      return;
    }
  } else {
    const int s = row / n_lrows, i = row - s * n_lrows;
    const int f = min(max(first[s], 0), m);
    if (i < f || i > min(m, n_lrows - 1)) return;
  }
  scan_chunk<kSum, kVec, kNoise>(logits + (long long)row * vocab, vocab, chunk,
                                 &part[(long long)row * n_chunks + chunk], red,
                                 kNoise ? noise + (long long)row * vocab : nullptr, inv_t);
}

// Merge the chunk partials of rows r0 .. r0 + nr - 1 that `want(i)`:
// 8 lanes per row, up to 8 chunks per lane per round, one round of loads for
// vocabularies up to 64 chunks (262144 logits).  `sink(i, acc)` receives each merged row
// (called by one lane per row).
template <typename Want, typename Sink>
__device__ void merge_rows(const ScanPartial* part, int n_chunks, int r0, int nr, Want want, Sink sink) {
  constexpr int kLanes = 8;
  const int tid = threadIdx.x;
  const int sub = tid % kLanes;
  for (int i0 = 0; i0 < nr; i0 += kScanThreads / kLanes) {
    const int i = i0 + tid / kLanes;
    const bool use = i < nr && want(i);
    Acc t{kNegInf, INT_MAX, 0.f};
    for (int c0 = 0; c0 < n_chunks; c0 += 8 * kLanes) {
      ScanPartial p[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + sub + kLanes * u;
        p[u] = ScanPartial{kNegInf, INT_MAX, 0.f, 0};
        if (use && c < n_chunks) p[u] = part[(long long)(r0 + i) * n_chunks + c];
      }
      // max first over the lane's partials, then index and rescaled sums
      Acc r{p[0].m, INT_MAX, 0.f};
#pragma unroll
      for (int u = 1; u < 8; ++u) r.m = fmaxf(r.m, p[u].m);
      if (r.m != kNegInf) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (p[u].m == r.m) r.a = min(r.a, p[u].a);
          if (p[u].m != kNegInf) r.s += p[u].s * __builtin_amdgcn_exp2f((p[u].m - r.m) * kLog2e);
        }
      }
      t = c0 == 0 ? r : merge(t, r);   // one round for up to 64 chunks
    }
    // the same across the row's lanes
    const float M = lanes_max<kLanes>(t.m);
    const int a_row = lanes_min<kLanes>(t.m == M ? t.a : INT_MAX);
    const float s_row = lanes_sum<kLanes>(t.m == kNegInf ? 0.f : t.s * __builtin_amdgcn_exp2f((t.m - M) * kLog2e));
    if (use && sub == 0) sink(i, Acc{M, a_row, s_row});
  }
}

// sum_v exp(l_v - mx) over one row by the whole workgroup, independent of
// the order of the terms: each float64 term t (in [0, 1]) is cut to
// floor(t 2^100), held as three 34-bit limbs that add without carries (a
// limb sum stays below 2^52 for any vocabulary under 2^18), and the total
// is rounded once to float64.  Two rows whose logits are permutations of
// each other therefore get the same sum, bit for bit.
constexpr int kFixBits = 100;

__device__ inline void add_term(double t, unsigned long long (&l)[3]) {
  const double x = ldexp(t, kFixBits);                 // exact
  const double h2 = floor(ldexp(x, -68));
  const double r1 = x - ldexp(h2, 68);                 // exact: the low bits of x
  const double h1 = floor(ldexp(r1, -34));
  const double r0 = r1 - ldexp(h1, 34);                // exact
  l[2] += (unsigned long long)h2;
  l[1] += (unsigned long long)h1;
  l[0] += (unsigned long long)r0;                      // r0 >= 0: truncation is floor
}

// (l0 + l1 2^34 + l2 2^68) 2^-100, rounded once to nearest (ties to even).
__device__ inline double limbs_to_double(const unsigned long long (&l)[3]) {
  const unsigned long long lo = l[0] + (l[1] << 34);
  const unsigned long long hi = (l[1] >> 30) + (l[2] << 4) + (lo < l[0] ? 1ull : 0ull);
  if (hi == 0) return ldexp((double)lo, -kFixBits);    // u64 -> f64 rounds once
  const int sh = 64 - __builtin_clzll(hi);             // 1 .. 54: the total is below 2^118
  unsigned long long top = (hi << (64 - sh)) | (lo >> sh);
  top |= (lo & ((1ull << sh) - 1)) != 0 ? 1ull : 0ull; // sticky bit, far below the rounding bit
  return ldexp((double)top, sh - kFixBits);
}

__device__ double row_sum_f64(const float* rowp, int vocab, float mx, unsigned long long* red) {
  const int tid = threadIdx.x;
  const double m = (double)mx;
  unsigned long long l[3] = {0, 0, 0};
  for (int v = tid; v < vocab; v += kScanThreads) add_term(exp((double)rowp[v] - m), l);
#pragma unroll
  for (int k = 0; k < 3; ++k) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) l[k] += __shfl_xor(l[k], off, 64);
  }
  if ((tid & 63) == 0) {
#pragma unroll
    for (int k = 0; k < 3; ++k) red[3 * (tid >> 6) + k] = l[k];
  }
  __syncthreads();
  unsigned long long t[3] = {0, 0, 0};
#pragma unroll
  for (int w = 0; w < kScanThreads / 64; ++w) {
#pragma unroll
    for (int k = 0; k < 3; ++k) t[k] += red[3 * w + k];
  }
  __syncthreads();
  return limbs_to_double(t);
}

// Workgroup reductions: wave shuffles, then one LDS slot per wave and a
// single barrier.  Each call site passes its own slots.
__device__ inline int block_sum(int v, int* slots) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  if ((threadIdx.x & 63) == 0) slots[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < kScanThreads / 64; ++w) t += slots[w];
  return t;
}

__device__ inline void block_min2(double& a, double& b, double* slots) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    a = fmin(a, __shfl_xor(a, off, 64));
    b = fmin(b, __shfl_xor(b, off, 64));
  }
  if ((threadIdx.x & 63) == 0) {
    slots[2 * (threadIdx.x >> 6)] = a;
    slots[2 * (threadIdx.x >> 6) + 1] = b;
  }
  __syncthreads();
  a = slots[0];
  b = slots[1];
#pragma unroll
  for (int w = 1; w < kScanThreads / 64; ++w) {
    a = fmin(a, slots[2 * w]);
    b = fmin(b, slots[2 * w + 1]);
  }
}

enum : unsigned char { kInE = 1, kRefined = 2, kNeedRefine = 4 };

struct SelectSmem {
  double cf[BC_MAX_BLOCK_ROWS];     // confidence; -inf for rows outside E
  float mrow[BC_MAX_BLOCK_ROWS];
  int tok[BC_MAX_BLOCK_ROWS];
  int rank[BC_MAX_BLOCK_ROWS];
  unsigned char st[BC_MAX_BLOCK_ROWS];
  unsigned long long key[64];        // one-wave path: rank keys of rows 0 .. 63
  unsigned long long red[3 * (kScanThreads / 64)];
  int cnt[2][kScanThreads / 64];
  double lohi[2][2 * (kScanThreads / 64)];
  int done;
};

// A double held by lane `lane` (wave-uniform), in every lane.
__device__ inline double readlane_f64(double v, int lane) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), lane);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Decisions of a block of at most 64 rows by wave 0 alone, lane i owning
// row i, when no float64 refine is needed: counts are ballots; ranks by
// (confidence desc, row asc) come from 64-bit integer keys, broadcast from
// LDS and compared once per row -- the float32 confidence's bits (monotone for positive values)
// above the complemented row index, rows outside E keyed 0 -- and, with no
// refined row in the block, every row carrying the same relative error band,
// the extreme of (c - e) over the top k and of (c + e) over the rest sit at
// ranks k - 1 and k.  Ranking in float32 is exact wherever it is used: the
// cut is accepted only when the float64 confidences at ranks k - 1 and k
// differ by more than the band, which dwarfs float32 rounding (rows that
// round to one float32 are ordered by row, and if they meet at the cut the
// check fails).  Returns false, having written nothing, when a row is
// inside the threshold band or the cut is not certain; the caller then
// takes the workgroup-wide path, which refines.
__device__ bool decide_one_wave(const UnmaskArgs& a, int b, int r0, int nb, double tau, int mode_b, int div_b,
                                uint8_t* masked, int* tokens, float* conf, SelectSmem& sm) {
  const int i = threadIdx.x;
  const bool inE = i < nb && (sm.st[i] & kInE);
  const double c = inE ? sm.cf[i] : -__builtin_huge_val();
  if (__ballot(inE && fabs(c - tau) <= kBand * c)) return false;
  const unsigned long long eb = __ballot(inE), ab = __ballot(inE && c > tau);
  const int nE = __popcll(eb), nA = __popcll(ab);
  int k;
  if (mode_b == BC_UNMASK_SEMI) {
    k = nA;
  } else {
    const int fb = (nE + div_b - 1) / div_b;
    k = min(nE, max(nA, fb));
  }
  const int how = k == 0 ? 0 : k == nE ? 1 : k == nA ? 2 : 3;
  int rk = 0;
  if (how == 3) {
    const uint32_t kc = inE ? __float_as_uint((float)c) : 0u;
    const unsigned long long key = ((unsigned long long)kc << 32) | (uint32_t)(63 - i);
    sm.key[i] = key;
    __builtin_amdgcn_s_waitcnt(0xc07f);        // lgkmcnt 0: every lane's key written
    __builtin_amdgcn_wave_barrier();
#pragma unroll 8
    for (int q = 0; q < nb; ++q) rk += sm.key[q] > key;   // broadcast reads
    // 1 <= k < nE, so ranks k - 1 and k are both rows of E
    const unsigned long long at0 = __ballot(inE && rk == k - 1), at1 = __ballot(inE && rk == k);
    if (!at0 || !at1) return false;
    const double c0 = readlane_f64(c, __builtin_ctzll(at0)), c1 = readlane_f64(c, __builtin_ctzll(at1));
    const double lo = c0 - kBand * c0, hi = c1 + kBand * c1;
    if (!(lo > hi)) return false;
  }
  if (inE) {
    const int r = r0 + i;
    const bool take = how == 1 || (how == 2 && c > tau) || (how == 3 && rk < k);
    if (take) {
      tokens[r] = sm.tok[i];
      masked[r] = 0;
    }
    if (conf) conf[r] = (float)c;
  }
  if (i == 0) a.n_commit[b] = k;
  return true;
}

// Decisions of block b, one workgroup.  Thread t owns rows t, t + 256, ...
// after the merge, so only the few workgroup reductions need barriers.
template <bool kDyn>
__global__ __launch_bounds__(kScanThreads) void unmask_decide_kernel(const UnmaskArgs a) {
  __shared__ SelectSmem sm;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  // the block's rows and rule: from the arguments, or from a device-resident
  // plan, whose flags and tokens sit at its row0 (blocks past its count idle)
  int r0, nb, mode_b, div_b, ro = 0;
  if constexpr (kDyn) {   // (uniform values: readfirstlane tells the compiler)
    if (b >= __builtin_amdgcn_readfirstlane(a.dyn->n)) return;
    r0 = __builtin_amdgcn_readfirstlane(a.dyn->blk_off[b]);
    nb = __builtin_amdgcn_readfirstlane(a.dyn->blk_off[b + 1]) - r0;
    mode_b = __builtin_amdgcn_readfirstlane(a.dyn->mode[b]);
    div_b = __builtin_amdgcn_readfirstlane(a.dyn->n_div[b]);
    ro = __builtin_amdgcn_readfirstlane(a.dyn->row0);
  } else {
    r0 = a.blk_off[b];
    nb = a.blk_off[b + 1] - r0;
  }
  uint8_t* const masked = kDyn ? a.masked + ro : a.masked;
  int* const tokens = kDyn ? a.tokens + ro : a.tokens;
  float* const conf = kDyn && a.conf ? a.conf + ro : a.conf;
  const double tau = (double)a.threshold;
  // The argument fields the merge and the decisions need, loaded in one
  // burst at kernel start: left to itself the compiler loads each next to
  // its first use, one scalar round trip after another (measured: section
  // decode +1.3%).  The block's mode and n are read early too: their
  // latency overlaps the merge.
  asm volatile("" ::"s"(a.masked), "s"(a.part), "s"(a.n_chunks), "s"(a.tokens), "s"(a.conf), "s"(a.n_commit),
               "s"(a.threshold));
  if constexpr (!kDyn) {
    mode_b = a.mode[b];
    div_b = a.n_div[b];
  }

  // The masked flags go to LDS, then every row's chunk partials are merged
  // (the flag stores wait for their loads first; holding the flags in
  // registers across the merge to share one round of loads measured slower).
  // Partials of revealed rows were not written by the scan and are dropped
  // below.
  for (int i = tid; i < nb; i += kScanThreads) sm.st[i] = masked[r0 + i] != 0 ? kInE : 0;
  merge_rows(a.part, a.n_chunks, r0, nb, [](int) { return true; },
             [&](int i, const Acc& t) {
               sm.cf[i] = 1.0 / (double)t.s;
               sm.tok[i] = t.a;
               sm.mrow[i] = t.m;
             });
  __syncthreads();
  if (nb <= 64) {
    if (tid < 64) {
      const bool ok = decide_one_wave(a, b, r0, nb, tau, mode_b, div_b, masked, tokens, conf, sm);
      if (tid == 0) sm.done = ok;
    }
    __syncthreads();
    if (sm.done) return;
  }
  for (int i = tid; i < nb; i += kScanThreads) {
    if (!(sm.st[i] & kInE)) {
      sm.cf[i] = -__builtin_huge_val();
    } else if (fabs(sm.cf[i] - tau) <= kBand * sm.cf[i]) {
      sm.st[i] |= kNeedRefine;   // threshold decision inside the band
    }
  }
  __syncthreads();

  // Re-take marked rows in float64; `any` is a workgroup-uniform flag.
  auto refine_marked = [&](bool any) {
    if (!any) return;
    for (int i = 0; i < nb; ++i) {
      if (!(sm.st[i] & kNeedRefine)) continue;      // uniform: st[] is shared
      const double s = row_sum_f64(a.logits + (long long)(r0 + i) * a.vocab, a.vocab, sm.mrow[i], sm.red);
      if (tid == 0) {
        sm.cf[i] = 1.0 / s;
        sm.st[i] = (unsigned char)((sm.st[i] & ~kNeedRefine) | kRefined);
      }
      __syncthreads();
    }
  };
  int my_mark = 0, my_e = 0, my_a = 0;
  for (int i = tid; i < nb; i += kScanThreads) {
    my_mark |= (sm.st[i] & kNeedRefine) != 0;
    my_e += (sm.st[i] & kInE) != 0;
  }
  refine_marked(__syncthreads_or(my_mark));
  for (int i = tid; i < nb; i += kScanThreads) my_a += (sm.st[i] & kInE) && sm.cf[i] > tau;
  const int packed = block_sum(my_e | (my_a << 16), sm.cnt[0]);
  const int nE = packed & 0xffff, nA = packed >> 16;
  int k;
  if (mode_b == BC_UNMASK_SEMI) {
    k = nA;
  } else {
    const int fb = (nE + div_b - 1) / div_b;
    k = min(nE, max(nA, fb));
  }

  // 0: nothing, 1: all of E, 2: exactly A, 3: top-k by rank
  const int how = k == 0 ? 0 : k == nE ? 1 : k == nA ? 2 : 3;
  if (how == 3) {
    // Rank with the current confidences; the cut is certain when the lowest
    // possible value inside the top k exceeds the highest possible value
    // outside it (refined rows carry no error).  Otherwise re-take the rows
    // whose error interval reaches across the cut in float64 and rank again.
    for (int guard = 0; guard <= nb; ++guard) {
      double lo = __builtin_huge_val(), hi_neg = __builtin_huge_val();
      for (int i = tid; i < nb; i += kScanThreads) {
        if (!(sm.st[i] & kInE)) continue;
        const double ci = sm.cf[i];
        int rk = 0;
#pragma unroll 8
        for (int q = 0; q < nb; ++q) {       // rows outside E hold -inf and never count
          const double cq = sm.cf[q];
          rk += cq > ci || (cq == ci && q < i);
        }
        sm.rank[i] = rk;
        const double e = (sm.st[i] & kRefined) ? 0.0 : kBand * ci;
        if (rk < k) lo = fmin(lo, ci - e);
        else hi_neg = fmin(hi_neg, -(ci + e));
      }
      block_min2(lo, hi_neg, sm.lohi[guard & 1]);
      const double hi = -hi_neg;
      if (lo > hi) break;
      int my_new = 0;
      for (int i = tid; i < nb; i += kScanThreads) {
        if (!(sm.st[i] & kInE) || (sm.st[i] & kRefined)) continue;
        const double c = sm.cf[i];
        const double e = kBand * c;
        if ((sm.rank[i] < k && c - e <= hi) || (sm.rank[i] >= k && c + e >= lo)) {
          sm.st[i] |= kNeedRefine;
          my_new = 1;
        }
      }
      if (!__syncthreads_or(my_new)) break;   // every row at the cut is exact: ranks decide
      refine_marked(true);
    }
  }

  for (int i = tid; i < nb; i += kScanThreads) {
    if (!(sm.st[i] & kInE)) continue;
    const int r = r0 + i;
    bool take = false;
    if (how == 1) take = true;
    else if (how == 2) take = sm.cf[i] > tau;
    else if (how == 3) take = sm.rank[i] < k;
    if (take) {
      tokens[r] = sm.tok[i];
      masked[r] = 0;
    }
    if (conf) conf[r] = (float)sm.cf[i];
  }
  if (tid == 0) a.n_commit[b] = k;
}

__global__ __launch_bounds__(kScanThreads) void verify_decide_kernel(const VerifyArgs a) {
  __shared__ int s_k;
  __shared__ int toks[BC_MAX_SCAN_ROWS];
  const int s = blockIdx.x, tid = threadIdx.x;
  asm volatile("" ::"s"(a.part), "s"(a.n_chunks), "s"(a.n_lrows), "s"(a.m), "s"(a.draft), "s"(a.fixed),
               "s"(a.accept_len), "s"(a.bonus));   // one burst of argument loads, as in the unmask decision
  const int f = min(max(a.first[s], 0), a.m);
  const int last_row = min(a.m, a.n_lrows - 1);     // rows f .. last_row were scanned
  const int nr = last_row - f + 1;                  // may be 0 (f == m == n_lrows)
  if (tid == 0) s_k = a.m;
  merge_rows(a.part, a.n_chunks, s * a.n_lrows + f, max(nr, 0), [](int) { return true; },
             [&](int i, const Acc& t) { toks[i] = t.a; });
  __syncthreads();
  for (int i = tid; i < a.m - f; i += kScanThreads) {
    const int r = f + i;
    const bool pass = (a.fixed && a.fixed[(long long)s * a.m + r]) || toks[i] == a.draft[(long long)s * a.m + r];
    if (!pass) atomicMin(&s_k, r);
  }
  __syncthreads();
  if (tid == 0) {
    const int k = s_k;
    a.accept_len[s] = k - f;
    a.bonus[s] = k < a.n_lrows ? toks[k - f] : -1;
  }
}

}  // namespace

hipError_t launch_scan(const float* logits, int n_rows, int vocab, const uint8_t* row_mask, bool with_sum,
                       ScanPartial* part, hipStream_t stream, const DevPlan* dyn) {
  const dim3 grid(scan_chunks(vocab), n_rows);
  const int nc = scan_chunks(vocab);
  const bool vec = vocab % 4 == 0;
  if (dyn) {   // the device-resident plan's instantiations (the unmask's scan)
    if (vec)
      hipLaunchKernelGGL((scan_kernel<0, true, true, false, true>), grid, dim3(kScanThreads), 0, stream, logits, vocab,
                         nc, part, row_mask, nullptr, 0, 0, nullptr, 1.f, dyn);
    else
      hipLaunchKernelGGL((scan_kernel<0, true, false, false, true>), grid, dim3(kScanThreads), 0, stream, logits,
                         vocab, nc, part, row_mask, nullptr, 0, 0, nullptr, 1.f, dyn);
    return hipGetLastError();
  }
  if (with_sum && vec)
    hipLaunchKernelGGL((scan_kernel<0, true, true>), grid, dim3(kScanThreads), 0, stream, logits, vocab, nc, part,
                       row_mask, nullptr, 0, 0);
  else if (with_sum)
    hipLaunchKernelGGL((scan_kernel<0, true, false>), grid, dim3(kScanThreads), 0, stream, logits, vocab, nc, part,
                       row_mask, nullptr, 0, 0);
  else if (vec)
    hipLaunchKernelGGL((scan_kernel<0, false, true>), grid, dim3(kScanThreads), 0, stream, logits, vocab, nc, part,
                       row_mask, nullptr, 0, 0);
  else
    hipLaunchKernelGGL((scan_kernel<0, false, false>), grid, dim3(kScanThreads), 0, stream, logits, vocab, nc, part,
                       row_mask, nullptr, 0, 0);
  return hipGetLastError();
}

hipError_t launch_unmask_decide(const UnmaskArgs& a, hipStream_t stream) {
  if (a.dyn)   // the device-resident plan's instantiation
    hipLaunchKernelGGL(unmask_decide_kernel<true>, dim3(a.n_blk), dim3(kScanThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(unmask_decide_kernel<false>, dim3(a.n_blk), dim3(kScanThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
  const dim3 grid(a.n_chunks, a.n_seq * a.n_lrows);
  const bool vec = a.vocab % 4 == 0;
  if (a.noise && vec)
    hipLaunchKernelGGL((scan_kernel<1, false, true, true>), grid, dim3(kScanThreads), 0, stream, a.logits, a.vocab,
                       a.n_chunks, a.part, nullptr, a.first, a.n_lrows, a.m, a.noise, a.inv_temperature);
  else if (a.noise)
    hipLaunchKernelGGL((scan_kernel<1, false, false, true>), grid, dim3(kScanThreads), 0, stream, a.logits,
                       a.vocab, a.n_chunks, a.part, nullptr, a.first, a.n_lrows, a.m, a.noise, a.inv_temperature);
  else if (vec)
    hipLaunchKernelGGL((scan_kernel<1, false, true>), grid, dim3(kScanThreads), 0, stream, a.logits, a.vocab,
                       a.n_chunks, a.part, nullptr, a.first, a.n_lrows, a.m);
  else
    hipLaunchKernelGGL((scan_kernel<1, false, false>), grid, dim3(kScanThreads), 0, stream, a.logits, a.vocab,
                       a.n_chunks, a.part, nullptr, a.first, a.n_lrows, a.m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(verify_decide_kernel, dim3(a.n_seq), dim3(kScanThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bc
