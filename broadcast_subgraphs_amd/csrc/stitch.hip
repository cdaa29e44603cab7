// Stitched memory-intensive subgraphs: row softmax, row LayerNorm (no affine),
// and pow -> broadcast -> add -> row softmax, each as ONE kernel.
//
// Every value has a home at the level of the hierarchy its dependency needs
// ([AStitch] "Four stitching schemes"):
//  * one-to-one elementwise chains stay in VGPRs (Local);
//  * reductions go thread -> wave (lane exchange) -> LDS (one reused scratch)
//    ([ComFuse] Stage-Stream Execution Model, reduce phase, Fig. 4);
//  * the per-row power value v_i^p is computed once per row per workgroup and
//    shared through LDS (Regional), never recomputed per element
//    ([AStitch] "What people did before", the power -> broadcast -> add case);
//  * rows wider than a workgroup holds are split over S workgroups that
//    aggregate through global memory with an in-kernel join (Global;
//    [AStitch] "Adaptive thread mapping", task splitting; [ComFuse] inter-CTA
//    level with every member reading all partials, the peer-to-peer mode).
//
// Stage chaining with bypass ([ComFuse] Fig. 3): the loaded fragments stay in
// registers across every reduction; each reduction's broadcast result drives
// the next stage without reloading or recomputing the inputs.
#include "dev.hpp"
#include "kernels.hpp"

namespace cf {

namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;

// Two LDS slots, used alternately by consecutive reductions, so one barrier
// per reduction suffices (the slot a reduction writes was last read before the
// previous reduction's barrier).  O(1) space however many reductions chain.
template <class Op, int LPR, int BLOCK = kBlock>
__device__ __forceinline__ float row_reduce(float v, float* red, int& slot, int group, int wave_in_row) {
  if constexpr (LPR <= kWave) {
    return group_reduce<Op, LPR>(v);
  } else {
    constexpr int WPR = LPR / kWave;  // waves per row
    constexpr int RPW = BLOCK / LPR;  // rows per workgroup
    v = group_reduce<Op, kWave>(v);
    float* s = red + slot * (BLOCK / kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) s[group * WPR + wave_in_row] = v;
    __syncthreads();
    float r = s[group * WPR];
#pragma unroll
    for (int w = 1; w < WPR; ++w) r = Op::op(r, s[group * WPR + w]);
    slot ^= 1;
    (void)RPW;
    return r;
  }
}

template <int W>
__device__ __forceinline__ void load_frag(float (&d)[W], const float* p) {
  if constexpr (W == 4) {
    float4 t = ld4_stream(p);
    d[0] = t.x; d[1] = t.y; d[2] = t.z; d[3] = t.w;
  } else {
    d[0] = __builtin_nontemporal_load(p);
  }
}

template <int W>
__device__ __forceinline__ void store_frag(float* p, const float (&d)[W]) {
  if constexpr (W == 4) {
    st4_stream(p, make_float4(d[0], d[1], d[2], d[3]));
  } else {
    __builtin_nontemporal_store(d[0], p);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Rows held inside one workgroup of BLOCK lanes.  A row is owned by a group
// of LPR lanes (packed BLOCK/LPR rows per workgroup when LPR < BLOCK; a
// workgroup of up to 1024 lanes owns a wide row whole, with no
// cross-workgroup exchange); lane q of the group holds
// fragments v*LPR + q (v < NV) of W floats each, so a wave's loads are
// contiguous.  Each lane keeps RPI rows in flight (vertical packing: a
// workgroup walks row blocks with a grid stride).
// ---------------------------------------------------------------------------
template <int OP, int LPR, int NV, int W, int RPI, int BLOCK = kBlock>
__global__ __launch_bounds__(BLOCK) void k_rows(RowArgs a) {
  constexpr int RPW = BLOCK / LPR;
  constexpr int WPR = LPR > kWave ? LPR / kWave : 1;
  __shared__ float red[2 * (BLOCK / kWave)];
  __shared__ float pv_lds[2][RPI * RPW];

  const int t = threadIdx.x;
  const int group = t / LPR;
  const int q = t % LPR;
  const int wave_in_row = (t % LPR) / kWave;
  const int64_t rows = a.rows, cols = a.cols;
  const int64_t rows_per_iter = (int64_t)RPW * RPI;
  const int64_t nblk = (rows + rows_per_iter - 1) / rows_per_iter;
  int slot = 0;
  int pvbuf = 0;
  (void)WPR;

  for (int64_t rb = blockIdx.x; rb < nblk; rb += gridDim.x) {
    float x[RPI][NV][W];
    bool rv[RPI];
    // ---- fragment loads (all in flight before any reduction)
#pragma unroll
    for (int r = 0; r < RPI; ++r) {
      const int64_t row = (rb * RPI + r) * RPW + group;
      rv[r] = row < rows;
      const float* xr = a.x + row * cols;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int64_t c0 = (int64_t)(v * LPR + q) * W;
        if (rv[r] && c0 < cols) {
          load_frag<W>(x[r][v], xr + c0);
        } else {
#pragma unroll
          for (int e = 0; e < W; ++e) x[r][v][e] = is_norm(OP) ? 0.0f : -INFINITY;
        }
      }
    }

    if constexpr (OP == kPowSoftmax) {
      // Regional scheme: v_i^p once per row per workgroup, broadcast via LDS.
      if (t < RPI * RPW) {
        const int64_t row = (rb * RPI + t / RPW) * RPW + (t % RPW);
        pv_lds[pvbuf][t] = row < rows ? powf(a.v[row], a.p) : 0.0f;
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < RPI; ++r) {
        const float pv = pv_lds[pvbuf][r * RPW + group];
        const int64_t row = (rb * RPI + r) * RPW + group;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int64_t c0 = (int64_t)(v * LPR + q) * W;
          const bool ok = rv[r] && c0 < cols;
#pragma unroll
          for (int e = 0; e < W; ++e) x[r][v][e] = ok ? x[r][v][e] + pv : -INFINITY;
          if (a.y_pre != nullptr && ok) store_frag<W>(a.y_pre + row * cols + c0, x[r][v]);
        }
      }
      pvbuf ^= 1;
    }

    if constexpr (OP == kSoftmax || OP == kPowSoftmax) {
      // stage 1: row max (base-2 domain: t = x * log2 e)
      float m[RPI];
#pragma unroll
      for (int r = 0; r < RPI; ++r) {
        float mm = -INFINITY;
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
          for (int e = 0; e < W; ++e) {
            x[r][v][e] *= kLog2e;
            mm = fmaxf(mm, x[r][v][e]);
          }
        m[r] = row_reduce<OpMax, LPR, BLOCK>(mm, red, slot, group, wave_in_row);
      }
      // stage 2: exp and row sum; exp values bypass into stage 3 in registers
      float inv[RPI];
#pragma unroll
      for (int r = 0; r < RPI; ++r) {
        float s = 0.0f;
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
          for (int e = 0; e < W; ++e) {
            const float ev = __builtin_amdgcn_exp2f(x[r][v][e] - m[r]);
            x[r][v][e] = ev;
            s += ev;
          }
        inv[r] = 1.0f / row_reduce<OpSum, LPR, BLOCK>(s, red, slot, group, wave_in_row);
      }
      // stage 3: broadcast divide and store
#pragma unroll
      for (int r = 0; r < RPI; ++r) {
        if (!rv[r]) continue;
        const int64_t row = (rb * RPI + r) * RPW + group;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int64_t c0 = (int64_t)(v * LPR + q) * W;
          if (c0 < cols) {
#pragma unroll
            for (int e = 0; e < W; ++e) x[r][v][e] *= inv[r];
            store_frag<W>(a.y + row * cols + c0, x[r][v]);
          }
        }
      }
    } else {  // the norms: LayerNorm (affine or not), RMSNorm (mean held at 0)
      const float inv_n = 1.0f / (float)cols;
      // gain / bias fragments of the lane's columns, loaded beside x (one round trip)
      constexpr bool GAIN = OP == kLayerNormAffine || OP == kRmsNorm, BIAS = OP == kLayerNormAffine;
      float gv[NV][W], bv[NV][W];
      if constexpr (GAIN) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int64_t c0 = (int64_t)(v * LPR + q) * W;
          if (a.gamma != nullptr && c0 < cols) {
            load_frag<W>(gv[v], a.gamma + c0);
          } else {
#pragma unroll
            for (int e = 0; e < W; ++e) gv[v][e] = 1.0f;
          }
          if constexpr (BIAS) {
            if (c0 < cols) {
              load_frag<W>(bv[v], a.beta + c0);
            } else {
#pragma unroll
              for (int e = 0; e < W; ++e) bv[v][e] = 0.0f;
            }
          }
        }
      }
      float mu[RPI];
#pragma unroll
      for (int r = 0; r < RPI; ++r) {
        if constexpr (OP == kRmsNorm) {
          mu[r] = 0.0f;
        } else {
          float s = 0.0f;
#pragma unroll
          for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int e = 0; e < W; ++e) s += x[r][v][e];
          mu[r] = row_reduce<OpSum, LPR, BLOCK>(s, red, slot, group, wave_in_row) * inv_n;
        }
      }
      float rs[RPI];
#pragma unroll
      for (int r = 0; r < RPI; ++r) {
        float s = 0.0f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int64_t c0 = (int64_t)(v * LPR + q) * W;
          const bool ok = c0 < cols;
#pragma unroll
          for (int e = 0; e < W; ++e) {
            const float c = ok ? x[r][v][e] - mu[r] : 0.0f;
            x[r][v][e] = c;
            s = fmaf(c, c, s);
          }
        }
        const float var = row_reduce<OpSum, LPR, BLOCK>(s, red, slot, group, wave_in_row) * inv_n;
        rs[r] = rsqrtf(var + a.eps);
      }
#pragma unroll
      for (int r = 0; r < RPI; ++r) {
        if (!rv[r]) continue;
        const int64_t row = (rb * RPI + r) * RPW + group;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int64_t c0 = (int64_t)(v * LPR + q) * W;
          if (c0 < cols) {
#pragma unroll
            for (int e = 0; e < W; ++e) {
              float o = x[r][v][e] * rs[r];
              if constexpr (GAIN) o *= gv[v][e];
              if constexpr (BIAS) o += bv[v][e];
              x[r][v][e] = o;
            }
            store_frag<W>(a.y + row * cols + c0, x[r][v]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Rows split over S workgroups (task splitting).  Logical item i = (row, s)
// with row = i / S, s = i % S covers columns [s*slice, min((s+1)*slice, cols)).
// Workgroup g handles items g, g+G, ... ; G is a multiple of S, so the S
// members of a row run in the same round, and the host guarantees the grid is
// resident at once.  Members publish partials, join, then every member reads
// all S partials and combines them in member order (deterministic).
// ---------------------------------------------------------------------------
template <int OP, int NV, int W>
__global__ __launch_bounds__(kBlock) void k_rows_split(RowArgs a) {
  __shared__ float red[2 * kWaves];
  __shared__ float bc[4];
  const int t = threadIdx.x;
  const int wave_in_row = t / kWave;
  int slot = 0;
  const int64_t rows = a.rows, cols = a.cols;
  const int S = a.S;
  const uint32_t G = gridDim.x;
  const int64_t items = rows * S;
  const uint32_t g = xcd_local_id(blockIdx.x, G);

  for (int64_t it = g; it < items; it += G) {
    const int64_t row = it / S;
    const int s = (int)(it % S);
    const int64_t cbeg = (int64_t)s * a.slice;
    const int64_t cend = min(cols, cbeg + a.slice);
    const float* xr = a.x + row * cols;

    float x[NV][W];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int64_t c0 = cbeg + (int64_t)(v * kBlock + t) * W;
      if (c0 < cend) {
        load_frag<W>(x[v], xr + c0);
      } else {
#pragma unroll
        for (int e = 0; e < W; ++e) x[v][e] = is_norm(OP) ? 0.0f : -INFINITY;
      }
    }

    float part0, part1, part2 = 0.0f;  // published partials of this member
    if constexpr (OP == kSoftmax || OP == kPowSoftmax) {
      float pv = 0.0f;
      if constexpr (OP == kPowSoftmax) {
        if (t == 0) bc[0] = powf(a.v[row], a.p);  // once per row per workgroup
        __syncthreads();
        pv = bc[0];
      }
      float mm = -INFINITY;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int64_t c0 = cbeg + (int64_t)(v * kBlock + t) * W;
        const bool ok = c0 < cend;
        if constexpr (OP == kPowSoftmax) {
#pragma unroll
          for (int e = 0; e < W; ++e) x[v][e] = ok ? x[v][e] + pv : -INFINITY;
          if (a.y_pre != nullptr && ok) store_frag<W>(a.y_pre + row * cols + c0, x[v]);
        }
#pragma unroll
        for (int e = 0; e < W; ++e) {
          x[v][e] *= kLog2e;
          mm = fmaxf(mm, x[v][e]);
        }
      }
      const float m = row_reduce<OpMax, kBlock>(mm, red, slot, 0, wave_in_row);
      float sl = 0.0f;
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < W; ++e) {
          const float ev = __builtin_amdgcn_exp2f(x[v][e] - m);
          x[v][e] = ev;
          sl += ev;
        }
      const float l = row_reduce<OpSum, kBlock>(sl, red, slot, 0, wave_in_row);
      part0 = m;
      part1 = l;
    } else {
      const float n_loc = cend > cbeg ? (float)(cend - cbeg) : 0.0f;
      float mean_loc = 0.0f;  // RMSNorm: the mean is held at 0 throughout
      if constexpr (OP != kRmsNorm) {
        float sx = 0.0f;
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
          for (int e = 0; e < W; ++e) sx += x[v][e];
        mean_loc = row_reduce<OpSum, kBlock>(sx, red, slot, 0, wave_in_row) / fmaxf(n_loc, 1.0f);
      }
      float sq = 0.0f;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int64_t c0 = cbeg + (int64_t)(v * kBlock + t) * W;
        const bool ok = c0 < cend;
#pragma unroll
        for (int e = 0; e < W; ++e) {
          const float c = ok ? x[v][e] - mean_loc : 0.0f;
          x[v][e] = c;
          sq = fmaf(c, c, sq);
        }
      }
      const float m2 = row_reduce<OpSum, kBlock>(sq, red, slot, 0, wave_in_row);
      part0 = n_loc;
      part1 = mean_loc;
      part2 = m2;
    }

    // ---- global level: publish, join, read all members' partials
    float4* P = reinterpret_cast<float4*>(a.partials) + (size_t)row * S;
    if (t == 0) {
      st_dev4(P + s, make_float4(part0, part1, part2, 0.0f));
      wait_stores();
      join_arrive_and_wait(a.joins + g / S, (uint32_t)S, a.err);  // members share g / S every round
    }
    __syncthreads();
    // Partials are read with device-scope loads, 8 in flight per batch.
    if constexpr (OP == kSoftmax || OP == kPowSoftmax) {
      float M = -INFINITY, L = 0.0f;
      for (int k0 = 0; k0 < S; k0 += 8) {  // 8 partials in flight per batch
        float4 q[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) q[k] = k0 + k < S ? ld_dev4(P + k0 + k) : make_float4(-INFINITY, 0.f, 0.f, 0.f);
#pragma unroll
        for (int k = 0; k < 8; ++k) M = fmaxf(M, q[k].x);
      }
      for (int k0 = 0; k0 < S; k0 += 8) {
        float4 q[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) q[k] = k0 + k < S ? ld_dev4(P + k0 + k) : make_float4(-INFINITY, 0.f, 0.f, 0.f);
#pragma unroll
        for (int k = 0; k < 8; ++k) L += q[k].x == -INFINITY ? 0.0f : q[k].y * __builtin_amdgcn_exp2f(q[k].x - M);
      }
      const float f = (part0 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(part0 - M)) / L;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int64_t c0 = cbeg + (int64_t)(v * kBlock + t) * W;
        if (c0 < cend) {
#pragma unroll
          for (int e = 0; e < W; ++e) x[v][e] *= f;
          store_frag<W>(a.y + row * cols + c0, x[v]);
        }
      }
    } else {
      // Chan's pairwise merge of (count, mean, M2), members in order.
      float n = 0.0f, mean = 0.0f, M2 = 0.0f;
      for (int k0 = 0; k0 < S; k0 += 8) {
        float4 q[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) q[k] = k0 + k < S ? ld_dev4(P + k0 + k) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float nb = q[k].x;
          if (nb == 0.0f) continue;
          const float nn = n + nb;
          const float d = q[k].y - mean;
          mean += d * (nb / nn);
          M2 += q[k].z + d * d * (n * nb / nn);
          n = nn;
        }
      }
      const float rs = rsqrtf(M2 / (float)cols + a.eps);
      const float shift = part1 - mean;  // this member's values are x - mean_loc
      constexpr bool GAIN = OP == kLayerNormAffine || OP == kRmsNorm, BIAS = OP == kLayerNormAffine;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int64_t c0 = cbeg + (int64_t)(v * kBlock + t) * W;
        if (c0 < cend) {
          float gv[W], bv[W];
          if (GAIN && a.gamma != nullptr) {
            load_frag<W>(gv, a.gamma + c0);
          } else {
#pragma unroll
            for (int e = 0; e < W; ++e) gv[e] = 1.0f;
          }
          if (BIAS) {
            load_frag<W>(bv, a.beta + c0);
          } else {
#pragma unroll
            for (int e = 0; e < W; ++e) bv[e] = 0.0f;
          }
#pragma unroll
          for (int e = 0; e < W; ++e) x[v][e] = fmaf((x[v][e] + shift) * rs, gv[e], bv[e]);
          store_frag<W>(a.y + row * cols + c0, x[v]);
        }
      }
    }
    __syncthreads();  // LDS slots and bc[] are reused by the next item
  }
}

// ---------------------------------------------------------------- dispatch

template <int OP, int W>
static hipError_t launch_rows_w(const RowPlan& pl, const RowArgs& a, hipStream_t st) {
  dim3 grid(pl.grid), block(kBlock);
  // Split plans first: they share (lpr, nv, rpi) with in-workgroup plans.
  if (pl.split > 1) {
#define CF_SPLIT(NV)                                                                        \
  if (pl.nv == NV) {                                                                        \
    hipLaunchKernelGGL((k_rows_split<OP, NV, W>), grid, block, 0, st, a);                   \
    return hipGetLastError();                                                               \
  }
    CF_SPLIT(1) CF_SPLIT(2) CF_SPLIT(4) CF_SPLIT(8) CF_SPLIT(16)
#undef CF_SPLIT
    return hipErrorInvalidConfiguration;
  }
#define CF_ROWS(LPR, NV, RPI)                                                               \
  if (pl.block == kBlock && pl.lpr == LPR && pl.nv == NV && pl.rpi == RPI) {                \
    hipLaunchKernelGGL((k_rows<OP, LPR, NV, W, RPI>), grid, block, 0, st, a);               \
    return hipGetLastError();                                                               \
  }
  CF_ROWS(4, 1, 4) CF_ROWS(8, 1, 4) CF_ROWS(16, 1, 4) CF_ROWS(32, 1, 4) CF_ROWS(64, 1, 4)
  CF_ROWS(4, 1, 2) CF_ROWS(8, 1, 2) CF_ROWS(16, 1, 2) CF_ROWS(32, 1, 2) CF_ROWS(64, 1, 2)
  CF_ROWS(4, 1, 1) CF_ROWS(8, 1, 1) CF_ROWS(16, 1, 1) CF_ROWS(32, 1, 1) CF_ROWS(64, 1, 1)
  CF_ROWS(8, 1, 8)
  CF_ROWS(64, 2, 1) CF_ROWS(64, 4, 1)
  CF_ROWS(128, 1, 1) CF_ROWS(128, 2, 1) CF_ROWS(128, 4, 1)
  CF_ROWS(256, 1, 1) CF_ROWS(256, 2, 1) CF_ROWS(256, 4, 1) CF_ROWS(256, 8, 1) CF_ROWS(256, 16, 1)
#undef CF_ROWS
  // one wide row per workgroup of 512 or 1024 lanes
#define CF_WIDE(BLOCK, NV)                                                                  \
  if (pl.block == BLOCK && pl.lpr == BLOCK && pl.nv == NV && pl.rpi == 1) {                 \
    hipLaunchKernelGGL((k_rows<OP, BLOCK, NV, W, 1, BLOCK>), grid, dim3(BLOCK), 0, st, a);  \
    return hipGetLastError();                                                               \
  }
  CF_WIDE(512, 8) CF_WIDE(512, 16) CF_WIDE(1024, 4) CF_WIDE(1024, 8)
#undef CF_WIDE
  return hipErrorInvalidConfiguration;
}

template <int W>
static hipError_t launch_rows_op(int op, const RowPlan& pl, const RowArgs& a, hipStream_t st) {
  switch (op) {
    case kSoftmax: return launch_rows_w<kSoftmax, W>(pl, a, st);
    case kLayerNorm: return launch_rows_w<kLayerNorm, W>(pl, a, st);
    case kPowSoftmax: return launch_rows_w<kPowSoftmax, W>(pl, a, st);
    case kLayerNormAffine: return launch_rows_w<kLayerNormAffine, W>(pl, a, st);
    case kRmsNorm: return launch_rows_w<kRmsNorm, W>(pl, a, st);
  }
  return hipErrorInvalidConfiguration;
}

hipError_t launch_rows(int op, const RowPlan& pl, const RowArgs& a, hipStream_t st) {
  return pl.w == 4 ? launch_rows_op<4>(op, pl, a, st) : launch_rows_op<1>(op, pl, a, st);
}

// Occupancy (resident workgroups per CU) of the split kernel for a plan.
hipError_t rows_split_occupancy(int op, const RowPlan& pl, int* per_cu) {
#define CF_OCC(OPV, NV, WV)                                                                 \
  if (op == OPV && pl.nv == NV && pl.w == WV)                                               \
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, k_rows_split<OPV, NV, WV>, kBlock, 0);
#define CF_OCC_NV(OPV, WV) CF_OCC(OPV, 1, WV) CF_OCC(OPV, 2, WV) CF_OCC(OPV, 4, WV) CF_OCC(OPV, 8, WV) CF_OCC(OPV, 16, WV)
  CF_OCC_NV(kSoftmax, 4) CF_OCC_NV(kLayerNorm, 4) CF_OCC_NV(kPowSoftmax, 4)
  CF_OCC_NV(kSoftmax, 1) CF_OCC_NV(kLayerNorm, 1) CF_OCC_NV(kPowSoftmax, 1)
  CF_OCC_NV(kLayerNormAffine, 4) CF_OCC_NV(kRmsNorm, 4) CF_OCC_NV(kLayerNormAffine, 1) CF_OCC_NV(kRmsNorm, 1)
#undef CF_OCC_NV
#undef CF_OCC
  return hipErrorInvalidConfiguration;
}

}  // namespace cf
