// Token permutation between the frame-major order of the model and an
// anchor-first temporal-major order used for temporal heads (patches in
// raster order, or block by block)
// ("Accelerating Spatio-Temporal Attention for Video Diffusion on TPUs",
// ainews.tenesys.com, list "Co się zmieniło?", item 5: reordering tokens so a
// patch's frames are adjacent speeds up temporal heads).
//
// Both directions are gathers: every destination row reads one source row, so
// stores are fully contiguous and loads are whole rows (head_dim * 2 bytes).
// Each thread moves 16 bytes per chunk; a wave moves 4 rows (d = 128) or 8
// (d = 64) per chunk.  The stores are non-temporal (the destination is
// written once and not read by this kernel): 5.1 -> 6.4 TB/s at 75,600
// tokens x 5 heads x d128.  The kernel is bound by HBM bandwidth.

#include "internal.hpp"

namespace svattn {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // 16-byte chunks per thread, loads issued before stores

__global__ __launch_bounds__(kThreads) void perm_index_kernel(Geo g, int order, int32_t* perm, int32_t* inv) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= g.N) return;
  const bool fm = order == SVATTN_FRAME_MAJOR;
  perm[t] = fm ? t : tm_to_fm(g, order, t);
  if (inv) inv[t] = fm ? t : fm_to_tm(g, order, t);
}

// CPR_SHIFT: log2(16-byte chunks per row).
template <int CPR_SHIFT>
__global__ __launch_bounds__(kThreads) void permute_kernel(Geo g, int order, FastDiv divN,
                                                           const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                           uint32_t n_chunks, int to_tm) {
  const uint32_t base = (blockIdx.x * kUnroll) * kThreads + threadIdx.x;
  uint4 val[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t c = base + u * kThreads;
    if (c < n_chunks) {
      const uint32_t row = c >> CPR_SHIFT;
      const uint32_t head = divN.div(row);
      const uint32_t pos = row - head * (uint32_t)g.N;
      const uint32_t srow = head * (uint32_t)g.N +
                            (uint32_t)(to_tm ? tm_to_fm(g, order, (int)pos) : fm_to_tm(g, order, (int)pos));
      val[u] = src[((size_t)srow << CPR_SHIFT) + (c & ((1u << CPR_SHIFT) - 1u))];
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t c = base + u * kThreads;
    if (c < n_chunks) {
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 w = {val[u].x, val[u].y, val[u].z, val[u].w};
      __builtin_nontemporal_store(w, (u32x4*)&dst[c]);
    }
  }
}

}  // namespace

hipError_t launch_perm_index(const Geo& g, int order, int32_t* perm, int32_t* inv, hipStream_t st) {
  hipLaunchKernelGGL(perm_index_kernel, dim3((g.N + kThreads - 1) / kThreads), dim3(kThreads), 0, st, g, order,
                     perm, inv);
  return hipGetLastError();
}

hipError_t launch_permute(const Geo& g, int order, int heads, int head_dim, const void* src, void* dst,
                          bool to_tm, hipStream_t st) {
  const int shift = head_dim == 128 ? 4 : 3;
  const uint64_t n_chunks = ((uint64_t)heads * g.N) << shift;
  const uint32_t per_block = kThreads * kUnroll;
  const dim3 grid((unsigned)((n_chunks + per_block - 1) / per_block));
  const FastDiv divN((uint32_t)g.N);
  if (shift == 4)
    hipLaunchKernelGGL(permute_kernel<4>, grid, dim3(kThreads), 0, st, g, order, divN, (const uint4*)src,
                       (uint4*)dst, (uint32_t)n_chunks, (int)to_tm);
  else
    hipLaunchKernelGGL(permute_kernel<3>, grid, dim3(kThreads), 0, st, g, order, divN, (const uint4*)src,
                       (uint4*)dst, (uint32_t)n_chunks, (int)to_tm);
  return hipGetLastError();
}

}  // namespace svattn
