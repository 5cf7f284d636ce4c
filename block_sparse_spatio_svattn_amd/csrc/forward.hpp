// Block-sparse flash-attention forward for gfx950 (CDNA4), bf16 MFMA.
//
// What it computes ("Accelerating Spatio-Temporal Attention for Video
// Diffusion on TPUs", aihirek.info): softmax attention restricted to the
// kept query-key pairs of a spatial or temporal head with a first-frame
// anchor (section "A Sparse VideoGen a figyelmi fejeket osztályozza"),
// visiting only non-empty tiles, with a mask-free path for full tiles and
// coordinate masking only on boundary tiles (section "A TPU-kernel
// kialakítása döntőnek bizonyult", paragraphs 2-3).
//
// Work decomposition.  One workgroup owns one (head, q-tile) of
// BQ = NW * QG * 32 queries; each of its NW waves owns QG groups of 32
// queries and keeps their Q fragments in registers for the whole loop.  The
// workgroup walks the q-tile's list of non-empty k-tiles; every k-tile's K and
// V (BK keys) are staged through LDS, double-buffered, with the next tile's
// global loads in flight while the current one is computed.
//
// Layouts.  Scores are computed transposed, S^T = K Q^T, with the
// 32x32x16 bf16 MFMA: K (A operand) comes from LDS, Q^T (B operand) from
// registers.  In the accumulator layout lane l holds query l % 32 and 16 of the
// 32 keys of a key block, so a query's running max and sum stay inside one
// lane pair (l, l ^ 32) -- one permlane32 swap per tile instead of a
// cross-lane tree.  The same registers, converted to bf16, are directly the B
// operand of O^T += V^T P^T: the 8 keys a lane supplies per 16-key step are
// the keys its accumulator registers hold.  V is therefore stored transposed
// in LDS with bits 2 and 3 of each key's position swapped, so the A operand
// (V^T) of a lane is one 16-byte read.  K rows and V^T rows are padded by 16
// bytes so the 16-byte LDS reads of 8 consecutive lanes hit distinct banks.
//
// Softmax.  exp2 with the scale folded into one FMA (p = 2^(s*c - m*c),
// c = scale*log2 e); masked scores are -inf.  The running max m is only
// moved when a new score exceeds it by more than 8 in log2 units, so most
// tiles skip rescaling the accumulator (values stay below 2^8 before
// normalisation, well inside fp32/bf16 range); the result differs only by
// rounding.  P is rounded to bf16 for the PV product; the row sum uses the
// fp32 values.
#pragma once

#include "internal.hpp"

namespace svattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <int D, int BK, int NW, int QG>
struct FwdCfg {
  static constexpr int NT = NW * 64;
  static constexpr int BQ = NW * QG * 32;
  static constexpr int KS = D + 8;   // bf16 per K row in LDS (16-byte pad)
  static constexpr int VS = BK + 8;  // bf16 per V^T row in LDS
  static constexpr int K_ELEMS = BK * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int BUF = K_ELEMS + V_ELEMS;     // bf16 per stage
  static constexpr int K_CHUNKS = BK * D / 8;       // 16-byte chunks of a K tile
  static constexpr int K_ITERS = (K_CHUNKS + NT - 1) / NT;
  static constexpr int V_QUADS = BK * D / 32;       // 4 keys x 8 dims
  static constexpr int V_ITERS = (V_QUADS + NT - 1) / NT;
  static constexpr int LDS_BYTES = 2 * BUF * 2 + 2 * BK * 4;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr float kNegBig = -1.0e30f;        // initial running max (finite)

__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Position of key k (0 <= k < BK) inside a V^T row: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

// Packed patch coordinates (y << 16 | x) of a key position, or a far-away
// value for positions >= N.
__device__ __forceinline__ int key_coord(const Geo& g, int order, int key) {
  if (key >= g.N) return 0x7fff7fff;
  const int p = patch_of(g, order, key);
  const int y = (int)g.divW.div((uint32_t)p);
  return (y << 16) | (p - y * g.W);
}

template <int D, int BK, int NW, int QG, bool BITS>
__global__ __launch_bounds__(NW * 64, 2) void fwd_kernel(const FwdArgs a) {
  using C = FwdCfg<D, BK, NW, QG>;
  static_assert(BK % 32 == 0 && D % 32 == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * C::BUF];
  __shared__ __attribute__((aligned(16))) int kcs[2][BK];

  // ---- work item: XCD-aware order (workgroup b runs on XCD b % 8) ----
  const int b = blockIdx.x;
  const int xcd = b & 7, s = b >> 3;
  const int item = ((s / a.chunk) * 8 + xcd) * a.chunk + (s % a.chunk);
  if (item >= a.n_items) return;
  const int slot = item / a.n_qt;
  const int qt = item - slot * a.n_qt;
  const HeadDesc hd = a.heads[slot];
  const Geo g = a.g;
  const int N = g.N;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const __bf16* __restrict__ Q = (const __bf16*)hd.q;
  const __bf16* __restrict__ K = (const __bf16*)hd.k;
  const __bf16* __restrict__ V = (const __bf16*)hd.v;
  const int q0 = qt * C::BQ + wave * (QG * 32);

  // ---- Q fragments (B operand of S^T = K Q^T) ----
  bf16x8 qf[QG][D / 16];
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) {
    const int qi = q0 + gq * 32 + l32;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      if (qi < N)
        qf[gq][ds] = *(const bf16x8*)(Q + (size_t)qi * D + ds * 16 + hh * 8);
      else
        qf[gq][ds] = bf16x8{};
    }
  }

  // ---- per-query mask parameters ----
  // spatial: kept non-anchor keys are [lo, lo + span); temporal: patch (y, x)
  int mq_a[QG], mq_b[QG];
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) {
    const int qi = min(q0 + gq * 32 + l32, N - 1);
    if (hd.kind == SVATTN_SPATIAL) {
      const int f = (int)g.divP.div((uint32_t)qi);
      const int flo = max(0, f - hd.window), fhi = min(g.F, f + hd.window + 1);
      mq_a[gq] = flo * g.P;
      mq_b[gq] = (fhi - flo) * g.P;
    } else {
      const int p = patch_of(g, hd.order, qi);
      const int y = (int)g.divW.div((uint32_t)p);
      mq_a[gq] = y;
      mq_b[gq] = p - y * g.W;
    }
  }
  const uint32_t* bits_row[QG];
  if constexpr (BITS) {
#pragma unroll
    for (int gq = 0; gq < QG; ++gq)
      bits_row[gq] = hd.bits + (size_t)min(q0 + gq * 32 + l32, N - 1) * a.words_per_row;
  }

  floatx16 acc[QG][D / 32];
#pragma unroll
  for (int gq = 0; gq < QG; ++gq)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[gq][db] = floatx16{};
  float m_run[QG], l_run[QG];
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) {
    m_run[gq] = kNegBig;
    l_run[gq] = 0.f;
  }
  const float c = hd.scale_log2;
  const bool need_kc = !BITS && hd.kind == SVATTN_TEMPORAL;

  // ---- tile list ----
  int e0, e1;
  if constexpr (BITS) {
    e0 = 0;
    e1 = a.n_kt;
  } else {
    e0 = hd.row_ptr[qt];
    e1 = hd.row_ptr[qt + 1];
  }

  // ---- staging registers for the next tile ----
  uint4 kreg[C::K_ITERS];
  uint4 vreg[C::V_ITERS][4];
  int kcreg = 0;

  auto tile_of = [&](int e) -> int {
    if constexpr (BITS) return e;
    else return hd.col[e];
  };

  auto global_load = [&](int kt) {
    const int key0 = kt * BK;
#pragma unroll
    for (int i = 0; i < C::K_ITERS; ++i) {
      const int cc = tid + i * C::NT;
      if (C::K_CHUNKS % C::NT == 0 || cc < C::K_CHUNKS) {
        const int row = cc / (D / 8), ch = cc % (D / 8);
        const int key = key0 + row;
        kreg[i] = key < N ? *(const uint4*)(K + (size_t)key * D + ch * 8) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < C::V_ITERS; ++i) {
      const int cc = tid + i * C::NT;
      if (C::V_QUADS % C::NT == 0 || cc < C::V_QUADS) {
        const int quad = cc % (BK / 4), dch = cc / (BK / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = key0 + quad * 4 + r;
          vreg[i][r] = key < N ? *(const uint4*)(V + (size_t)key * D + dch * 8) : make_uint4(0, 0, 0, 0);
        }
      }
    }
    if (need_kc && tid < BK) kcreg = key_coord(g, hd.order, key0 + tid);
  };

  auto lds_store = [&](int buf) {
    __bf16* Ks = smem + buf * C::BUF;
    __bf16* Vt = Ks + C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::K_ITERS; ++i) {
      const int cc = tid + i * C::NT;
      if (C::K_CHUNKS % C::NT == 0 || cc < C::K_CHUNKS) {
        const int row = cc / (D / 8), ch = cc % (D / 8);
        *(uint4*)(Ks + row * C::KS + ch * 8) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < C::V_ITERS; ++i) {
      const int cc = tid + i * C::NT;
      if (C::V_QUADS % C::NT == 0 || cc < C::V_QUADS) {
        const int quad = cc % (BK / 4), dch = cc / (BK / 4);
        const int pos = vt_pos(quad * 4);
        const uint32_t* r0 = (const uint32_t*)&vreg[i][0];
        const uint32_t* r1 = (const uint32_t*)&vreg[i][1];
        const uint32_t* r2 = (const uint32_t*)&vreg[i][2];
        const uint32_t* r3 = (const uint32_t*)&vreg[i][3];
#pragma unroll
        for (int w = 0; w < 4; ++w) {  // dims 2w, 2w+1 of this 8-dim chunk
          uint2 lo, hi;
          lo.x = (r0[w] & 0xffffu) | (r1[w] << 16);
          lo.y = (r2[w] & 0xffffu) | (r3[w] << 16);
          hi.x = (r0[w] >> 16) | (r1[w] & 0xffff0000u);
          hi.y = (r2[w] >> 16) | (r3[w] & 0xffff0000u);
          *(uint2*)(Vt + (dch * 8 + 2 * w) * C::VS + pos) = lo;
          *(uint2*)(Vt + (dch * 8 + 2 * w + 1) * C::VS + pos) = hi;
        }
      }
    }
    if (need_kc && tid < BK) kcs[buf][tid] = kcreg;
  };

  if (e0 < e1) {
    global_load(tile_of(e0));
    lds_store(0);
  }
  __syncthreads();

  for (int e = e0; e < e1; ++e) {
    const int buf = (e - e0) & 1;
    const int kt = tile_of(e);
    int cls;
    if constexpr (BITS) cls = SVATTN_TILE_BOUNDARY;
    else cls = hd.col_cls[e];
    if (e + 1 < e1) global_load(tile_of(e + 1));

    const __bf16* Ks = smem + buf * C::BUF;
    const __bf16* Vt = Ks + C::K_ELEMS;
    const int key0 = kt * BK;

    // ---- S^T = K Q^T ----
    floatx16 sacc[BK / 32][QG];
#pragma unroll
    for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
      for (int gq = 0; gq < QG; ++gq) sacc[kb][gq] = floatx16{};
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
#pragma unroll
      for (int kb = 0; kb < BK / 32; ++kb) {
        const bf16x8 ka = *(const bf16x8*)(Ks + (kb * 32 + l32) * C::KS + ds * 16 + hh * 8);
#pragma unroll
        for (int gq = 0; gq < QG; ++gq)
          sacc[kb][gq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[gq][ds], sacc[kb][gq], 0, 0, 0);
      }
    }

    // ---- mask: boundary tiles and the ragged last tile only ----
    const bool ragged = key0 + BK > N;
    if (cls == SVATTN_TILE_BOUNDARY || ragged) {
      if (BITS) {
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) {
#pragma unroll
          for (int kb = 0; kb < BK / 32; ++kb) {
            const uint32_t word = key0 + kb * 32 < N ? bits_row[gq][(key0 >> 5) + kb] : 0u;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int kk = 8 * (i / 4) + 4 * hh + (i % 4);
              const bool keep = ((word >> kk) & 1u) && (key0 + kb * 32 + kk < N);
              if (!keep) sacc[kb][gq][i] = -INFINITY;
            }
          }
        }
      } else if (hd.kind == SVATTN_SPATIAL) {
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) {
#pragma unroll
          for (int kb = 0; kb < BK / 32; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = key0 + kb * 32 + 8 * (i / 4) + 4 * hh + (i % 4);
              const bool keep = key < g.P || (uint32_t)(key - mq_a[gq]) < (uint32_t)mq_b[gq];
              if (!keep) sacc[kb][gq][i] = -INFINITY;
            }
          }
        }
      } else if (hd.kind == SVATTN_TEMPORAL) {
        const int r = hd.radius;
#pragma unroll
        for (int kb = 0; kb < BK / 32; ++kb) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int kk0 = kb * 32 + 8 * i4 + 4 * hh;
            const int4 kc4 = *(const int4*)&kcs[buf][kk0];
            const int kcv[4] = {kc4.x, kc4.y, kc4.z, kc4.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int key = key0 + kk0 + j;
              const int yk = kcv[j] >> 16, xk = kcv[j] & 0xffff;
#pragma unroll
              for (int gq = 0; gq < QG; ++gq) {
                const bool near = (uint32_t)(yk - mq_a[gq] + r) <= (uint32_t)(2 * r) &&
                                  (uint32_t)(xk - mq_b[gq] + r) <= (uint32_t)(2 * r);
                if (!(near || key < g.P)) sacc[kb][gq][i4 * 4 + j] = -INFINITY;
              }
            }
          }
        }
      } else {  // dense: only the key range
#pragma unroll
        for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + kb * 32 + 8 * (i / 4) + 4 * hh + (i % 4);
            if (key >= N)
#pragma unroll
              for (int gq = 0; gq < QG; ++gq) sacc[kb][gq][i] = -INFINITY;
          }
      }
    }

    // ---- online softmax ----
    bf16x8 pf[BK / 16][QG];
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][gq][i]);
      mx = max_xor32(mx);
      const float m_new = fmaxf(m_run[gq], mx);
      const bool need = (m_new - m_run[gq]) * c > kRescaleThreshold;
      if (__any(need)) {
        const float alpha = need ? __builtin_amdgcn_exp2f((m_run[gq] - m_new) * c) : 1.0f;
        if (need) m_run[gq] = m_new;
        l_run[gq] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[gq][db] *= alpha;
      }
      const float mc = m_run[gq] * c;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < BK / 32; ++kb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x8 p;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float v = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][gq][h * 8 + j], c, -mc));
            ls += v;
            p[j] = (__bf16)v;
          }
          pf[kb * 2 + h][gq] = p;
        }
      }
      l_run[gq] += ls;
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 va = *(const bf16x8*)(Vt + (db * 32 + l32) * C::VS + ks * 16 + hh * 8);
#pragma unroll
        for (int gq = 0; gq < QG; ++gq)
          acc[gq][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[ks][gq], acc[gq][db], 0, 0, 0);
      }
    }

    if (e + 1 < e1) lds_store(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, lse = m*scale + ln l ----
  __bf16* __restrict__ O = (__bf16*)hd.o;
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) {
    const int qi = q0 + gq * 32 + l32;
    const float l = sum_xor32(l_run[gq]);
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    if (qi < N) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = db * 32 + 8 * i4 + 4 * hh;
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          bf16x4 ov;
#pragma unroll
          for (int j = 0; j < 4; ++j) ov[j] = (__bf16)(acc[gq][db][i4 * 4 + j] * inv);
          *(bf16x4*)(O + (size_t)qi * D + d0) = ov;
        }
      }
      if (hd.lse && hh == 0)
        hd.lse[qi] =
            l > 0.f ? m_run[gq] * hd.scale + __logf(l) : -INFINITY;
    }
  }
}

template <int D, int BK, int NW, int QG, bool BITS>
hipError_t launch_fwd_cfg(const FwdArgs& a, hipStream_t st) {
  using C = FwdCfg<D, BK, NW, QG>;
  const int per_round = 8 * a.chunk;
  const int grid = ((a.n_items + per_round - 1) / per_round) * per_round;
  hipLaunchKernelGGL((fwd_kernel<D, BK, NW, QG, BITS>), dim3(grid), dim3(C::NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace svattn
