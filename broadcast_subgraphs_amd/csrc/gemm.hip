// bf16 MFMA GEMM whose epilogue runs a stitched stage DAG across output tiles.
//
// MainLoop ([ComFuse] Stage-Stream Execution Model, tile-level streaming):
// each workgroup of 4 waves (2 x 2) computes a BM x BN accumulator tile with
// v_mfma_f32_32x32x16_bf16, staging BK-deep operand tiles in a two-stage LDS
// ring fed through registers (the next stage's global loads are in flight
// while the current stage feeds the MFMAs; [ComFuse] B2BGEMM producer and
// multi-stage circular buffer).  LDS rows are XOR-swizzled so fragment reads
// are bank-conflict free.  A [M x K] is K-contiguous.  The right operand is
// either W [K x N] (N-contiguous; fragments come from the LDS transpose read
// ds_read_b64_tr_b16) or K [N x K] (K-contiguous; plain 16-byte reads).
//
// The MFMA is issued with the operands swapped (MFMA A = right operand,
// MFMA B = left operand) and with a fixed permutation of the right operand's
// columns, so that each lane's 16 accumulator values are 16 CONSECUTIVE
// columns of ONE output row.  Row reductions are therefore mostly
// thread-local, and epilogue loads/stores are 32-byte row segments.
//
// Epilogue ([ComFuse] Fig. 3 stage chain with bypass; inter-CTA level): the
// accumulator stays in registers through every stage.  Per-row statistics are
// reduced thread -> lane pair -> LDS (across the 2 column waves) -> across the
// tiles of the row group through global memory with an in-kernel join.  A
// persistent grid walks tiles in rounds that contain whole row groups, and the
// host sizes the grid to what is resident at once, so every join completes
// ([AStitch] "What it costs": barrier validity requires residency).  Each
// output element has exactly one owning tile ([sass2mlir] "Epilogue fusion").
#include "dev.hpp"
#include "kernels.hpp"

namespace cf {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr int kThreads = 256;

// 16-byte-chunk XOR swizzle for K-contiguous tiles [rows][BK]: 8 consecutive
// rows reading the same logical chunk hit 8 distinct 16-byte bank groups.
template <int BK>
__device__ __forceinline__ int swz(int row, int c) {
  constexpr int CPR = BK / 8;
  constexpr int RD = CPR >= 8 ? 1 : 8 / CPR;
  constexpr int MOD = CPR >= 8 ? 8 : CPR;
  return c ^ ((row / RD) % MOD);
}

// Byte-offset XOR for N-contiguous tiles [BK][BN]: the 4 k-rows a transpose
// read touches land 0, 16, 64 and 80 bytes apart modulo the bank width.
__device__ __forceinline__ int nn_mask(int k) { return ((k & 1) << 4) | (((k >> 1) & 1) << 6); }

// Output column (within a 32-column block) of MFMA row i under the permutation
// that makes lane (l >> 5) hold columns 16*(l>>5) .. 16*(l>>5)+15.
__device__ __forceinline__ int sigma(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

template <int BM, int BN, int BK, bool NN>
struct Tile {
  static constexpr int CPR = BK / 8;             // 16-byte chunks per K-row
  static constexpr int CA = BM * BK / 8 / kThreads;
  static constexpr int CB = BN * BK / 8 / kThreads;
  static constexpr int A_ELEMS = BM * BK;
  static constexpr int B_ELEMS = BN * BK;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;  // bf16 elements per LDS stage
  static_assert(CA * kThreads * 8 == BM * BK && CB * kThreads * 8 == BN * BK, "tile/threads");

  uint4 ra[CA];
  uint4 rb[CB];

  __device__ __forceinline__ void load(const GemmArgs& a, int64_t m0, int64_t n0, int64_t k0) {
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < CA; ++j) {
      const int id = j * kThreads + t;
      const int row = id / CPR, c = id % CPR;
      const int64_t gm = m0 + row, gk = k0 + 8 * c;
      ra[j] = (gm < a.M && gk < a.K) ? *reinterpret_cast<const uint4*>(a.A + gm * a.K + gk)
                                     : make_uint4(0, 0, 0, 0);
    }
    if constexpr (NN) {
      constexpr int CPRB = BN / 8;
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const int id = j * kThreads + t;
        const int k = id / CPRB, c = id % CPRB;
        const int64_t gk = k0 + k, gn = n0 + 8 * c;
        rb[j] = (gk < a.K && gn < a.N) ? *reinterpret_cast<const uint4*>(a.B + gk * a.N + gn)
                                       : make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const int id = j * kThreads + t;
        const int row = id / CPR, c = id % CPR;
        const int64_t gn = n0 + row, gk = k0 + 8 * c;
        rb[j] = (gn < a.N && gk < a.K) ? *reinterpret_cast<const uint4*>(a.B + gn * a.K + gk)
                                       : make_uint4(0, 0, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* st) const {
    const int t = threadIdx.x;
    uint16_t* As = st;
    uint16_t* Bs = st + A_ELEMS;
#pragma unroll
    for (int j = 0; j < CA; ++j) {
      const int id = j * kThreads + t;
      const int row = id / CPR, c = id % CPR;
      *reinterpret_cast<uint4*>(As + row * BK + 8 * swz<BK>(row, c)) = ra[j];
    }
    if constexpr (NN) {
      constexpr int CPRB = BN / 8;
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const int id = j * kThreads + t;
        const int k = id / CPRB, c = id % CPRB;
        char* rowp = reinterpret_cast<char*>(Bs) + k * (BN * 2);
        *reinterpret_cast<uint4*>(rowp + ((16 * c) ^ nn_mask(k))) = rb[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const int id = j * kThreads + t;
        const int row = id / CPR, c = id % CPR;
        *reinterpret_cast<uint4*>(Bs + row * BK + 8 * swz<BK>(row, c)) = rb[j];
      }
    }
  }
};

// One BK-deep stage of MFMAs from LDS.
template <int BM, int BN, int BK, bool NN, int RB, int CB>
__device__ __forceinline__ void mma_stage(const uint16_t* st, f32x16 (&acc)[RB][CB], int wm, int wn) {
  constexpr int WM = BM / 2, WN = BN / 2;
  const int lane = threadIdx.x & 63;
  const uint16_t* As = st;
  const uint16_t* Bs = st + BM * BK;
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    bf16x8_t bop[RB];  // left operand rows (MFMA B)
    bf16x8_t aop[CB];  // right operand columns (MFMA A)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = wm * WM + rb * 32 + (lane & 31);
      const int c = 2 * ks + (lane >> 5);
      bop[rb] = *reinterpret_cast<const bf16x8_t*>(As + row * BK + 8 * swz<BK>(row, c));
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      if constexpr (NN) {
        const int G = lane >> 4, L = lane & 15;
        const int e = L >> 2, cc = L & 3;
        const int kbase = 8 * (G >> 1);
        const int n = wn * WN + cb * 32 + 16 * (cc & 1) + 8 * (G & 1) + 4 * (cc >> 1);
        bf16x4_t h[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int k = ks * 16 + kbase + 4 * hh + e;
          const char* p = reinterpret_cast<const char*>(Bs) + k * (BN * 2) + ((2 * n) ^ nn_mask(k));
          h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
        }
        aop[cb] = __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
      } else {
        const int n = wn * WN + cb * 32 + sigma(lane & 31);
        const int c = 2 * ks + (lane >> 5);
        aop[cb] = *reinterpret_cast<const bf16x8_t*>(Bs + n * BK + 8 * swz<BK>(n, c));
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[cb], bop[rb], acc[rb][cb], 0, 0, 0);
  }
}

// Cross-wave (column halves) combine of per-row values through LDS.  red has
// 2 slots x 2 waves x BM floats; the slot alternates per call.
template <class Op, int BM, int RB>
__device__ __forceinline__ void tile_row_reduce(float (&v)[RB], float* red, int& slot, int wm, int wn) {
  constexpr int WM = BM / 2;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) v[rb] = Op::op(v[rb], __shfl_xor(v[rb], 32, kWave));
  float* s = red + slot * (2 * BM);
  if (lane < 32) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) s[wn * BM + wm * WM + rb * 32 + lane] = v[rb];
  }
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = wm * WM + rb * 32 + (lane & 31);
    v[rb] = Op::op(s[r], s[BM + r]);
  }
  slot ^= 1;
}

}  // namespace

template <int EPI, bool NN, int BM, int BN, int BK, int MINB>
__global__ __launch_bounds__(kThreads, MINB) void k_gemm(GemmArgs a) {
  using T = Tile<BM, BN, BK, NN>;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int RB = WM / 32, CB = WN / 32;
  __shared__ __align__(16) uint16_t lds[2 * T::STAGE];

  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int hl = lane >> 5, l32 = lane & 31;
  const int KT = (int)((a.K + BK - 1) / BK);
  const uint32_t G = gridDim.x;
  const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
  const uint32_t g = (EPI == kEpiStoreF32) ? blockIdx.x : xcd_local_id(blockIdx.x, G);

  for (int64_t tile = g; tile < tiles; tile += G) {
    const int64_t rowblk = tile / a.tiles_n;
    const int tn = (int)(tile % a.tiles_n);
    const int64_t m0 = rowblk * BM, n0 = (int64_t)tn * BN;

    f32x16 acc[RB][CB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.0f;

    // ------------------------------------------------------------ MainLoop
    T tl;
    tl.load(a, m0, n0, 0);
    tl.store(lds);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < KT) tl.load(a, m0, n0, (int64_t)(kt + 1) * BK);
      mma_stage<BM, BN, BK, NN, RB, CB>(lds + cur * T::STAGE, acc, wm, wn);
      if (kt + 1 < KT) tl.store(lds + (cur ^ 1) * T::STAGE);
      __syncthreads();
    }

    // lane's output coordinates: row(rb) = m0 + wm*WM + rb*32 + l32,
    // cols(cb) = n0 + wn*WN + cb*32 + 16*hl + [0, 16)
    if constexpr (EPI == kEpiStoreF32) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int64_t row = m0 + wm * WM + rb * 32 + l32;
        if (row >= a.M) continue;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int64_t col = n0 + wn * WN + cb * 32 + 16 * hl;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (col + 4 * q < a.N)
              st4_stream(a.Z + row * a.N + col + 4 * q,
                         make_float4(acc[rb][cb][4 * q], acc[rb][cb][4 * q + 1], acc[rb][cb][4 * q + 2],
                                     acc[rb][cb][4 * q + 3]));
        }
      }
    } else {
      // The staging ring is free now; reuse it as the epilogue's LDS scratch.
      float* red = reinterpret_cast<float*>(lds);        // 2 slots x 2 x BM
      float4* pub = reinterpret_cast<float4*>(red + 4 * BM);  // BM published partials
      float2* stat = reinterpret_cast<float2*>(pub + BM);     // BM combined statistics
      int slot = 0;
      const float n_tile = (float)(a.N - n0 < BN ? a.N - n0 : (int64_t)BN);

      bool colok[CB][2];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int64_t col = n0 + wn * WN + cb * 32 + 16 * hl;
        colok[cb][0] = col < a.N;
        colok[cb][1] = col + 8 < a.N;
      }

      float p0[RB], p1[RB], p2[RB];
      if constexpr (EPI == kEpiLN) {
        // stage 1: u = acc + bias_j + R_ij, kept in the accumulator registers
        float bv[CB][16];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int64_t col = n0 + wn * WN + cb * 32 + 16 * hl;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 b = colok[cb][q >> 1] ? *reinterpret_cast<const float4*>(a.bias + col + 4 * q)
                                               : make_float4(0.f, 0.f, 0.f, 0.f);
            bv[cb][4 * q] = b.x; bv[cb][4 * q + 1] = b.y; bv[cb][4 * q + 2] = b.z; bv[cb][4 * q + 3] = b.w;
          }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int64_t row = m0 + wm * WM + rb * 32 + l32;
          u32x4 rr[CB][2];
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            const int64_t col = n0 + wn * WN + cb * 32 + 16 * hl;
#pragma unroll
            for (int h = 0; h < 2; ++h)
              rr[cb][h] = (a.R != nullptr && row < a.M && colok[cb][h])
                              ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.R + row * a.N + col + 8 * h))
                              : u32x4{0u, 0u, 0u, 0u};
          }
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const uint32_t wv = rr[cb][r >> 3][(r & 7) >> 1];
              const float u = acc[rb][cb][r] + bv[cb][r] + ((r & 1) ? bf16_hi(wv) : bf16_lo(wv));
              acc[rb][cb][r] = colok[cb][r >> 3] ? u : 0.0f;
            }
          }
        }
        // stage 1 reduce: tile-local row mean
        float s[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          float v = 0.0f;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) v += acc[rb][cb][r];
          s[rb] = v;
        }
        tile_row_reduce<OpSum, BM, RB>(s, red, slot, wm, wn);
        float mt[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) mt[rb] = s[rb] / n_tile;
        // stage 2 reduce: tile-local sum of squared deviations (u stays in registers)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          float v = 0.0f;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float d = colok[cb][r >> 3] ? acc[rb][cb][r] - mt[rb] : 0.0f;
              v = fmaf(d, d, v);
            }
          s[rb] = v;
        }
        tile_row_reduce<OpSum, BM, RB>(s, red, slot, wm, wn);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          p0[rb] = n_tile;
          p1[rb] = mt[rb];
          p2[rb] = s[rb];
        }
      } else {  // kEpiSoftmax: s = scale * acc, base-2 domain
        const float sc = a.scale * kLog2e;
        float mx[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          float v = -INFINITY;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float sv = colok[cb][r >> 3] ? acc[rb][cb][r] * sc : -INFINITY;
              acc[rb][cb][r] = sv;
              v = fmaxf(v, sv);
            }
          mx[rb] = v;
        }
        tile_row_reduce<OpMax, BM, RB>(mx, red, slot, wm, wn);
        float l[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          float v = 0.0f;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float e = __builtin_amdgcn_exp2f(acc[rb][cb][r] - mx[rb]);
              acc[rb][cb][r] = e;  // bypass: exp values feed the final stage
              v += e;
            }
          l[rb] = v;
        }
        tile_row_reduce<OpSum, BM, RB>(l, red, slot, wm, wn);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          p0[rb] = mx[rb];
          p1[rb] = l[rb];
          p2[rb] = 0.0f;
        }
      }

      // ---------------------------------------------- global level: publish
      if (wn == 0 && hl == 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) pub[wm * WM + rb * 32 + l32] = make_float4(p0[rb], p1[rb], p2[rb], 0.f);
      }
      __syncthreads();
      if (w == 0) {
        float* P = a.partials;
        for (int r = lane; r < BM; r += kWave) {
          const int64_t row = m0 + r;
          if (row < a.M) {
            const float4 v = pub[r];
            float* d = P + ((size_t)row * a.tiles_n + tn) * 4;
            st_agent(d + 0, v.x);
            st_agent(d + 1, v.y);
            st_agent(d + 2, v.z);
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        // the members of a row group share g / tiles_n in every round
        if (lane == 0) join_arrive_and_wait(a.joins + g / a.tiles_n, (uint32_t)a.tiles_n, a.err);
      }
      __syncthreads();

      // every member combines all members' partials, in member order
      if (t < BM) {
        const int64_t row = m0 + t;
        float2 st2 = make_float2(0.f, 0.f);
        if (row < a.M) {
          const float* P = a.partials + (size_t)row * a.tiles_n * 4;
          if constexpr (EPI == kEpiLN) {
            float n = 0.f, mean = 0.f, M2 = 0.f;
            for (int k = 0; k < a.tiles_n; ++k) {
              const float nb = ld_agent(P + 4 * k), mb = ld_agent(P + 4 * k + 1), m2b = ld_agent(P + 4 * k + 2);
              const float nn = n + nb;
              const float d = mb - mean;
              mean += d * (nb / nn);
              M2 += m2b + d * d * (n * nb / nn);
              n = nn;
            }
            st2 = make_float2(mean, rsqrtf(M2 / (float)a.N + a.eps));
          } else {
            float M = -INFINITY;
            for (int k = 0; k < a.tiles_n; ++k) M = fmaxf(M, ld_agent(P + 4 * k));
            float L = 0.f;
            for (int k = 0; k < a.tiles_n; ++k) L += ld_agent(P + 4 * k + 1) * __builtin_amdgcn_exp2f(ld_agent(P + 4 * k) - M);
            st2 = make_float2(M, 1.0f / L);
          }
        }
        stat[t] = st2;
      }
      __syncthreads();

      // ------------------------------------------------ final stage + commit
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int rl = wm * WM + rb * 32 + l32;
        const int64_t row = m0 + rl;
        const float2 st2 = stat[rl];
        float fa, fb;  // LN: y = (acc - fb) * fa * gamma + beta; softmax: y = acc * fa
        if constexpr (EPI == kEpiLN) {
          fa = st2.y;
          fb = st2.x;
        } else {
          fa = __builtin_amdgcn_exp2f(p0[rb] - st2.x) * st2.y;
          fb = 0.f;
        }
        if (row >= a.M) continue;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int64_t col = n0 + wn * WN + cb * 32 + 16 * hl;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            if (!colok[cb][h]) continue;
            float o[8];
            if constexpr (EPI == kEpiLN) {
              const float4 g0 = *reinterpret_cast<const float4*>(a.gamma + col + 8 * h);
              const float4 g1 = *reinterpret_cast<const float4*>(a.gamma + col + 8 * h + 4);
              const float4 b0 = *reinterpret_cast<const float4*>(a.beta + col + 8 * h);
              const float4 b1 = *reinterpret_cast<const float4*>(a.beta + col + 8 * h + 4);
              const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
              const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
              for (int e = 0; e < 8; ++e) o[e] = fmaf((acc[rb][cb][8 * h + e] - fb) * fa, gg[e], bb[e]);
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) o[e] = acc[rb][cb][8 * h + e] * fa;
            }
            const u32x4 pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                              pack_bf16x2(o[6], o[7])};
            __builtin_nontemporal_store(pk, reinterpret_cast<u32x4*>(a.Y + row * a.N + col + 8 * h));
          }
        }
      }
    }
    __syncthreads();  // LDS is reused by the next tile's prologue
  }
}

// ---------------------------------------------------------------- dispatch

bool gemm_tile_config(int cfg, int* bm, int* bn, int* bk) {
  switch (cfg) {
    case 0: *bm = 256; *bn = 256; *bk = 64; return true;
    case 1: *bm = 128; *bn = 256; *bk = 32; return true;
    case 2: *bm = 128; *bn = 128; *bk = 64; return true;
    case 3: *bm = 256; *bn = 128; *bk = 64; return true;
    default: return false;
  }
}

template <int EPI, bool NN>
static hipError_t launch_gemm_t(const GemmPlan& pl, const GemmArgs& a, hipStream_t st, int* occ) {
#define CF_GEMM(CFG, BM, BN, BK, MINB)                                                             \
  if (pl.cfg == CFG) {                                                                             \
    if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, k_gemm<EPI, NN, BM, BN, BK, MINB>, kThreads, 0); \
    hipLaunchKernelGGL((k_gemm<EPI, NN, BM, BN, BK, MINB>), dim3(pl.grid), dim3(kThreads), 0, st, a); \
    return hipGetLastError();                                                                      \
  }
  CF_GEMM(0, 256, 256, 64, 1)
  CF_GEMM(1, 128, 256, 32, 2)
  CF_GEMM(2, 128, 128, 64, 2)
  CF_GEMM(3, 256, 128, 64, 1)
#undef CF_GEMM
  return hipErrorInvalidConfiguration;
}

static hipError_t gemm_dispatch(int epi, const GemmPlan& pl, const GemmArgs& a, hipStream_t st, int* occ) {
  if (epi == kEpiLN) return pl.nn ? launch_gemm_t<kEpiLN, true>(pl, a, st, occ) : hipErrorInvalidConfiguration;
  if (epi == kEpiSoftmax) return pl.nn ? hipErrorInvalidConfiguration : launch_gemm_t<kEpiSoftmax, false>(pl, a, st, occ);
  return pl.nn ? launch_gemm_t<kEpiStoreF32, true>(pl, a, st, occ) : launch_gemm_t<kEpiStoreF32, false>(pl, a, st, occ);
}

hipError_t launch_gemm(int epi, const GemmPlan& pl, const GemmArgs& a, hipStream_t st) {
  return gemm_dispatch(epi, pl, a, st, nullptr);
}

hipError_t gemm_occupancy(int epi, const GemmPlan& pl, int* per_cu) {
  return gemm_dispatch(epi, pl, GemmArgs{}, nullptr, per_cu);
}

}  // namespace cf
