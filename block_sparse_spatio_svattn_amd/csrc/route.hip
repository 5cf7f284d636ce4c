// Head routing: deviation of the spatial and temporal outputs from the dense
// output over the sampled query rows, and the mask with the smaller one
// ("Accelerating Spatio-Temporal Attention for Video Diffusion on TPUs",
// aihirek.info, section "A Sparse VideoGen a figyelmi fejeket osztályozza",
// paragraph 3).  The three outputs come from the attention forward run over
// the sampled q-tiles only, written compactly; this kernel reduces them.

#include "internal.hpp"

namespace svattn {
namespace {

constexpr int kRouteThreads = 256;

// One workgroup per head.  o_* are [heads, rows, d] bf16; rows past the
// valid count are ignored.  err[h] = {mean squared deviation of spatial,
// of temporal}; choice[h] = SVATTN_TEMPORAL iff its deviation is smaller.
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const uint16_t* o_dense, const uint16_t* o_spatial,
                                                              const uint16_t* o_temporal, int64_t per_head,
                                                              int64_t valid, float* err, int32_t* choice) {
  __shared__ float red[2][kRouteThreads / 64];
  const int h = blockIdx.x;
  const uint16_t* d = o_dense + h * per_head;
  const uint16_t* s = o_spatial + h * per_head;
  const uint16_t* t = o_temporal + h * per_head;
  float es = 0.f, et = 0.f;
  for (int64_t i = threadIdx.x; i < valid; i += kRouteThreads) {
    const float vd = __uint_as_float((uint32_t)d[i] << 16);
    const float vs = __uint_as_float((uint32_t)s[i] << 16) - vd;
    const float vt = __uint_as_float((uint32_t)t[i] << 16) - vd;
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
    float a = 0.f, b = 0.f;
    for (int w = 0; w < kRouteThreads / 64; ++w) {
      a += red[0][w];
      b += red[1][w];
    }
    a /= (float)valid;
    b /= (float)valid;
    err[2 * h] = a;
    err[2 * h + 1] = b;
    choice[h] = b < a ? SVATTN_TEMPORAL : SVATTN_SPATIAL;
  }
}

}  // namespace

hipError_t launch_route(const void* o_dense, const void* o_spatial, const void* o_temporal, int heads,
                        int64_t per_head, int64_t valid, float* err, int32_t* choice, hipStream_t st) {
  hipLaunchKernelGGL(route_kernel, dim3(heads), dim3(kRouteThreads), 0, st, (const uint16_t*)o_dense,
                     (const uint16_t*)o_spatial, (const uint16_t*)o_temporal, per_head, valid, err, choice);
  return hipGetLastError();
}

}  // namespace svattn
