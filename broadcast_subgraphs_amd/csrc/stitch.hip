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

// One pair reduction over the whole workgroup: lane butterfly, then the waves'
// pairs through LDS, merged in wave order by every lane (the same bits on every
// lane).  The caller's next use of `lds` is behind a later barrier.
template <int WAVES, class P>
__device__ __forceinline__ P block_reduce_pair(P p, P* lds, int wave) {
  p = wave_reduce(p);
  if constexpr (WAVES == 1) return p;
  if ((threadIdx.x & (kWave - 1)) == 0) lds[wave] = p;
  __syncthreads();
  P r = lds[0];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) {
    if constexpr (sizeof(P) == sizeof(SmPair)) r = sm_merge(r, lds[w]);
    else r = mom_merge(r, lds[w]);
  }
  return r;
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
    // pow-softmax: the rows' v, issued ahead of the fragment loads so v^p is
    // ready when they land
    float vrow = 0.0f;
    if constexpr (OP == kPowSoftmax) {
      if (t < RPI * RPW) {
        const int64_t row = (rb * RPI + t / RPW) * RPW + (t % RPW);
        if (row < rows) vrow = a.v[row];
      }
    }
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
      if (t < RPI * RPW) pv_lds[pvbuf][t] = powf(vrow, a.p);
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
// Rows split over S workgroups (task splitting).  Workgroup g is member
// s = g % S of group g / S for the whole launch; the group walks rows g / S,
// g / S + G / S, ... (G, a multiple of S, is resident at once), member s
// covering columns [s*slice, min((s+1)*slice, cols)) of each.
//
// Exchange ([AStitch] "Four stitching schemes", Global; [ComFuse] inter-CTA
// level, peer-to-peer): per row, each member publishes its two partials
// (softmax: max and sum in the base-2 domain; the norms: mean and M2 of its
// slice, whose count follows from the slice bounds) as tagged slots, one
// 64-bit store each; wave 0 takes every member's slots once they carry the
// row's tag (the value arrives with the tag: no arrival counter, no reload),
// and every lane merges them from LDS in member order (deterministic).  A
// slot is reused two rows later (double-buffered by row parity): before a
// member rewrites it, every member has published the next row, which it does
// only after taking this row's slots.  Across launches: before its first load
// each member clears its slots and arrives on the group's join word; it awaits
// the others before its first take, so the join overlaps the first loads, and
// no slot read in a launch holds a word from an earlier one (tags restart at
// 1, and a cleared slot carries tag 0).
// ---------------------------------------------------------------------------
template <int OP, int NV, int W, int BLOCK = kBlock>
__global__ __launch_bounds__(BLOCK) void k_rows_split(RowArgs a) {
  constexpr int WAVES = BLOCK / kWave;
  __shared__ SmPair red2[WAVES];
  __shared__ MomPair red3[WAVES];
  __shared__ float bc[4];
  __shared__ float pm[2][kMaxSplit];
  const int t = threadIdx.x;
  const int wave_in_row = t / kWave;
  const int64_t rows = a.rows, cols = a.cols;
  const int S = a.S;
  const uint32_t G = gridDim.x;
  const uint32_t g = xcd_local_id(blockIdx.x, G);
  const int s = (int)(g % (uint32_t)S);
  const int64_t grp = g / (uint32_t)S, groups = G / (uint32_t)S;
  uint64_t* const slots = a.slots + grp * (4 * S);  // [parity][field][member]
  uint64_t jold = 0;
  if (t == 0 && grp < rows) {  // (the planner gives every group a row)
#pragma unroll
    for (int k = 0; k < 4; ++k) slot_clear(slots + k * S + s);
    wait_stores();
    jold = join_arrive(a.joins + grp, (uint32_t)S);
  }
  const int64_t cbeg = (int64_t)s * a.slice;
  const int64_t cend = min(cols, cbeg + a.slice);
  uint32_t it_ = 0;

  for (int64_t row = grp; row < rows; row += groups, ++it_) {
    const float* xr = a.x + row * cols;
    float vrow = 0.0f;
    if constexpr (OP == kPowSoftmax) {
      if (t == 0) vrow = a.v[row];  // issued ahead of the row's loads, so v^p is ready when they land
    }
    float x[NV][W];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int64_t c0 = cbeg + (int64_t)(v * BLOCK + t) * W;
      if (c0 < cend) {
        load_frag<W>(x[v], xr + c0);
      } else {
#pragma unroll
        for (int e = 0; e < W; ++e) x[v][e] = is_norm(OP) ? 0.0f : -INFINITY;
      }
    }

    // ---- the member's statistics in ONE reduction (lane, wave, LDS): the
    // online (max, sum) pair, or (count, mean, M2)
    float part0, part1;  // this member's published partials
    float lane_ref;      // softmax: the lane's max; norms: the lane's mean
    if constexpr (OP == kSoftmax || OP == kPowSoftmax) {
      float pv = 0.0f;
      if constexpr (OP == kPowSoftmax) {
        if (t == 0) bc[0] = powf(vrow, a.p);  // once per row per workgroup
        __syncthreads();
        pv = bc[0];
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int64_t c0 = cbeg + (int64_t)(v * BLOCK + t) * W;
        const bool ok = c0 < cend;
        if constexpr (OP == kPowSoftmax) {
#pragma unroll
          for (int e = 0; e < W; ++e) x[v][e] = ok ? x[v][e] + pv : -INFINITY;
          if (a.y_pre != nullptr && ok) store_frag<W>(a.y_pre + row * cols + c0, x[v]);
        }
#pragma unroll
        for (int e = 0; e < W; ++e) {
          x[v][e] *= kLog2e;
          mloc = fmaxf(mloc, x[v][e]);
        }
      }
      const float ms = mloc == -INFINITY ? 0.0f : mloc;  // an all-masked lane keeps exp2(-inf) = 0
      float lloc = 0.0f;
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < W; ++e) {
          const float ev = __builtin_amdgcn_exp2f(x[v][e] - ms);
          x[v][e] = ev;
          lloc += ev;
        }
      const SmPair w = block_reduce_pair<WAVES>(SmPair{mloc, lloc}, red2, wave_in_row);
      part0 = w.m;
      part1 = w.l;
      lane_ref = mloc;
    } else {
      float nl = 0.0f, sx = 0.0f;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int64_t c0 = cbeg + (int64_t)(v * BLOCK + t) * W;
        if (c0 < cend) nl += (float)W;
#pragma unroll
        for (int e = 0; e < W; ++e) sx += x[v][e];
      }
      // RMSNorm: the mean is held at 0 throughout
      const float ml = (OP == kRmsNorm || nl == 0.0f) ? 0.0f : sx / nl;
      float sq = 0.0f;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int64_t c0 = cbeg + (int64_t)(v * BLOCK + t) * W;
        const bool ok = c0 < cend;
#pragma unroll
        for (int e = 0; e < W; ++e) {
          const float c = ok ? x[v][e] - ml : 0.0f;
          x[v][e] = c;
          sq = fmaf(c, c, sq);
        }
      }
      const MomPair w = block_reduce_pair<WAVES>(MomPair{nl, ml, sq}, red3, wave_in_row);
      part0 = w.mean;
      part1 = w.m2;
      lane_ref = ml;
    }

    // ---- global level: tagged slots, published and taken by wave 0.  The
    // first row waits for the launch join (every member's slots cleared)
    // before any lane takes a slot.
    const uint32_t tag = it_ + 1u;
    uint64_t* const sp = slots + (it_ & 1u) * (2 * S);
    if (it_ == 0) {
      if (t == 0) join_await(a.joins + grp, jold, (uint32_t)S, a.err);
      __syncthreads();
    }
    if (t < kWave) {
      if (t == 0) {
        slot_put(sp + s, tag, part0);
        slot_put(sp + S + s, tag, part1);
      }
      for (int q = t; q < S; q += kWave) slot_take2(sp + q, sp + S + q, tag, a.err, &pm[0][q], &pm[1][q]);
    }
    __syncthreads();
    if constexpr (OP == kSoftmax || OP == kPowSoftmax) {
      float M = -INFINITY, L = 0.0f;
      for (int q = 0; q < S; ++q) M = fmaxf(M, pm[0][q]);
      for (int q = 0; q < S; ++q) L += pm[0][q] == -INFINITY ? 0.0f : pm[1][q] * __builtin_amdgcn_exp2f(pm[0][q] - M);
      // this lane's exponentials are relative to its own max
      const float f = (lane_ref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(lane_ref - M)) / L;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int64_t c0 = cbeg + (int64_t)(v * BLOCK + t) * W;
        if (c0 < cend) {
#pragma unroll
          for (int e = 0; e < W; ++e) x[v][e] *= f;
          store_frag<W>(a.y + row * cols + c0, x[v]);
        }
      }
    } else {
      // Chan's pairwise merge of (count, mean, M2), members in order; member
      // q's count is the width of its slice
      float n = 0.0f, mean = 0.0f, M2 = 0.0f;
      for (int q = 0; q < S; ++q) {
        const int64_t qb = (int64_t)q * a.slice;
        const float nb = qb < cols ? (float)(min(cols, qb + a.slice) - qb) : 0.0f;
        if (nb == 0.0f) continue;
        const float nn = n + nb;
        const float d = pm[0][q] - mean;
        mean += d * (nb / nn);
        M2 += pm[1][q] + d * d * (n * nb / nn);
        n = nn;
      }
      const float rs = rsqrtf(M2 / (float)cols + a.eps);
      const float shift = lane_ref - mean;  // this lane's values are x minus its own mean
      constexpr bool GAIN = OP == kLayerNormAffine || OP == kRmsNorm, BIAS = OP == kLayerNormAffine;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int64_t c0 = cbeg + (int64_t)(v * BLOCK + t) * W;
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
    __syncthreads();  // LDS slots, bc[] and pm[] are reused by the next row
  }
}

// ---------------------------------------------------------------- dispatch

template <int OP, int W>
static hipError_t launch_rows_w(const RowPlan& pl, const RowArgs& a, hipStream_t st) {
  dim3 grid(pl.grid), block(kBlock);
  // Split plans first: they share (lpr, nv, rpi) with in-workgroup plans.
  // Members are 256-lane workgroups (up to 16 fragments per lane) or, for
  // many very wide rows, 1024-lane ones (up to 8).
  if (pl.split > 1) {
#define CF_SPLIT(BLK, NV)                                                                   \
  if (pl.block == BLK && pl.nv == NV) {                                                     \
    hipLaunchKernelGGL((k_rows_split<OP, NV, W, BLK>), grid, dim3(BLK), 0, st, a);          \
    return hipGetLastError();                                                               \
  }
    CF_SPLIT(kBlock, 1) CF_SPLIT(kBlock, 2) CF_SPLIT(kBlock, 4) CF_SPLIT(kBlock, 8) CF_SPLIT(kBlock, 16)
    if constexpr (OP != kLayerNormAffine) { CF_SPLIT(1024, 4) CF_SPLIT(1024, 8) }
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
  // one wide row per workgroup of 1024 lanes
#define CF_WIDE(BLOCK, NV)                                                                  \
  if (pl.block == BLOCK && pl.lpr == BLOCK && pl.nv == NV && pl.rpi == 1) {                 \
    hipLaunchKernelGGL((k_rows<OP, BLOCK, NV, W, 1, BLOCK>), grid, dim3(BLOCK), 0, st, a);  \
    return hipGetLastError();                                                               \
  }
  CF_WIDE(1024, 4) CF_WIDE(1024, 8)
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
  if (op == OPV && pl.nv == NV && pl.w == WV && pl.block == kBlock)                         \
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, k_rows_split<OPV, NV, WV>, kBlock, 0);
#define CF_OCC_WIDE(OPV, NV, WV)                                                            \
  if (op == OPV && pl.nv == NV && pl.w == WV && pl.block == 1024)                           \
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, k_rows_split<OPV, NV, WV, 1024>, 1024, 0);
#define CF_OCC_NV(OPV, WV) CF_OCC(OPV, 1, WV) CF_OCC(OPV, 2, WV) CF_OCC(OPV, 4, WV) CF_OCC(OPV, 8, WV) CF_OCC(OPV, 16, WV)
  CF_OCC_NV(kSoftmax, 4) CF_OCC_NV(kLayerNorm, 4) CF_OCC_NV(kPowSoftmax, 4)
  CF_OCC_NV(kSoftmax, 1) CF_OCC_NV(kLayerNorm, 1) CF_OCC_NV(kPowSoftmax, 1)
  CF_OCC_NV(kLayerNormAffine, 4) CF_OCC_NV(kRmsNorm, 4) CF_OCC_NV(kLayerNormAffine, 1) CF_OCC_NV(kRmsNorm, 1)
#define CF_OCC_W(OPV, WV) CF_OCC_WIDE(OPV, 4, WV) CF_OCC_WIDE(OPV, 8, WV)
  CF_OCC_W(kSoftmax, 4) CF_OCC_W(kLayerNorm, 4) CF_OCC_W(kPowSoftmax, 4) CF_OCC_W(kRmsNorm, 4)
  CF_OCC_W(kSoftmax, 1) CF_OCC_W(kLayerNorm, 1) CF_OCC_W(kPowSoftmax, 1) CF_OCC_W(kRmsNorm, 1)
#undef CF_OCC_W
#undef CF_OCC_WIDE
#undef CF_OCC_NV
#undef CF_OCC
  return hipErrorInvalidConfiguration;
}

}  // namespace cf
