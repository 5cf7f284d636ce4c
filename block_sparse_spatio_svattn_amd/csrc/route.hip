// Head routing: deviation of the spatial and temporal outputs from the dense
// output over the sampled query rows, and the mask with the smaller one
// ("Accelerating Spatio-Temporal Attention for Video Diffusion on TPUs",
// aihirek.info, section "A Sparse VideoGen a figyelmi fejeket osztályozza",
// paragraph 3).
//
// The three outputs come from one attention forward over the sampled q-tiles
// whose key lists are cut into splits (so that a few rows still fill the
// chip); each split leaves its rows normalised over its own keys together
// with their log-sum-exp.  Here the splits of a row are merged exactly as a
// softmax over their union: O = sum_s e^(lse_s - M) O_s / sum_s e^(lse_s - M),
// M = max_s lse_s; the merged row is rounded to bf16, as the forward's output
// would be, before the squared deviations are summed.

#include "internal.hpp"

namespace svattn {
namespace {

constexpr int kRouteThreads = kRouteMergeThreads;
constexpr int kColsPerThread = kRouteColsPerThread;

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float round_bf16(float x) { return (float)(__bf16)x; }

struct RouteParts {
  const float* o[3];
  const float* lse[3];
};

// Merged row (4 columns from c4) of mask m; rows of one (head, q-tile) are
// `rows` apart between splits.
__device__ __forceinline__ floatx4 merged(const RouteParts& p, int m, size_t row0, int64_t rows, int n_split,
                                         int head_dim, int c4) {
  const float* lse = p.lse[m] + row0;
  float mx = -INFINITY;
  for (int s = 0; s < n_split; ++s) mx = fmaxf(mx, lse[s * rows]);
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  if (mx == -INFINITY) return acc;  // no split keeps a key of this row
  float den = 0.f;
  const float* o = p.o[m] + row0 * head_dim + c4;
  for (int s = 0; s < n_split; ++s) {
    const float e = __expf(lse[s * rows] - mx);
    den += e;
    const floatx4 v = *(const floatx4*)(o + (size_t)s * rows * head_dim);
    acc += e * v;
  }
  return acc / den;
}

// Grid: heads * n_sel * (block_q / rows_per_block) workgroups; workgroup b
// covers rows_per_block rows of one (head, q-tile) and writes its two sums of
// squared deviations to perr[2 b], perr[2 b + 1].
__global__ __launch_bounds__(kRouteThreads) void route_merge_kernel(RouteParts p, int n_sel, int n_split,
                                                                    int block_q, int head_dim, float* perr) {
  __shared__ float red[2][kRouteThreads / 64];
  const int cpr = head_dim / kColsPerThread;  // threads per row
  const int rpb = kRouteThreads / cpr;         // rows per workgroup
  const int per_tile = block_q / rpb;
  const int b = blockIdx.x;
  const int ht = b / per_tile;                 // head * n_sel + q-tile rank
  const int r = (b - ht * per_tile) * rpb + threadIdx.x / cpr;
  const int c4 = (threadIdx.x % cpr) * kColsPerThread;
  // row r of split 0 of (head, q-tile) ht; split s is s * block_q rows further
  const size_t row0 = (size_t)ht * n_split * block_q + r;
  const floatx4 d = merged(p, 0, row0, block_q, n_split, head_dim, c4);
  const floatx4 sp = merged(p, 1, row0, block_q, n_split, head_dim, c4);
  const floatx4 tp = merged(p, 2, row0, block_q, n_split, head_dim, c4);
  float es = 0.f, et = 0.f;
#pragma unroll
  for (int j = 0; j < kColsPerThread; ++j) {
    const float vd = round_bf16(d[j]);
    const float vs = round_bf16(sp[j]) - vd;
    const float vt = round_bf16(tp[j]) - vd;
    es = __builtin_fmaf(vs, vs, es);
    et = __builtin_fmaf(vt, vt, et);
  }
  for (int off = 32; off > 0; off >>= 1) {
    es += __shfl_xor(es, off);
    et += __shfl_xor(et, off);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wave] = es;
    red[1][wave] = et;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = 0.f, c = 0.f;
    for (int w = 0; w < kRouteThreads / 64; ++w) {
      a += red[0][w];
      c += red[1][w];
    }
    perr[2 * b] = a;
    perr[2 * b + 1] = c;
  }
}

// One thread per head: the head's workgroup sums in a fixed order, the mean
// over its rows * head_dim values, and the choice (a tie goes to spatial).
__global__ __launch_bounds__(64) void route_choose_kernel(const float* perr, int heads, int blocks_per_head,
                                                          float count, float* err, int32_t* choice) {
  const int h = blockIdx.x * 64 + threadIdx.x;
  if (h >= heads) return;
  const float* pe = perr + (size_t)h * blocks_per_head * 2;
  float a = 0.f, c = 0.f;
  for (int i = 0; i < blocks_per_head; ++i) {
    a += pe[2 * i];
    c += pe[2 * i + 1];
  }
  a /= count;
  c /= count;
  err[2 * h] = a;
  err[2 * h + 1] = c;
  choice[h] = c < a ? SVATTN_TEMPORAL : SVATTN_SPATIAL;
}

}  // namespace

hipError_t launch_route(const float* const o[3], const float* const lse[3], int heads, int n_sel, int n_split,
                        int block_q, int head_dim, float* perr, float* err, int32_t* choice, hipStream_t st) {
  RouteParts p;
  for (int m = 0; m < 3; ++m) {
    p.o[m] = o[m];
    p.lse[m] = lse[m];
  }
  const int per_tile = block_q / route_rows_per_block(head_dim);
  const int blocks_per_head = n_sel * per_tile;
  hipLaunchKernelGGL(route_merge_kernel, dim3(heads * blocks_per_head), dim3(kRouteThreads), 0, st, p, n_sel,
                     n_split, block_q, head_dim, perr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float count = (float)n_sel * block_q * head_dim;  // exact: below 2^24
  hipLaunchKernelGGL(route_choose_kernel, dim3((heads + 63) / 64), dim3(64), 0, st, perr, heads, blocks_per_head,
                     count, err, choice);
  return hipGetLastError();
}

}  // namespace svattn
