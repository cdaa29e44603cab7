// bf16 MFMA GEMM whose epilogue runs a stitched stage DAG across output tiles.
//
// MainLoop ([ComFuse] Stage-Stream Execution Model, tile-level streaming;
// B2BGEMM producer with a multi-stage circular buffer): each workgroup of 4
// waves computes a BM x BN fp32 accumulator tile with v_mfma_f32_32x32x16_bf16.
// Operand tiles BK deep stream into a STAGES-deep LDS ring with direct
// global->LDS buffer loads (no VGPR staging; out-of-range chunks read as zero
// through the buffer descriptor's range check).  LDS rows are XOR-swizzled so
// the fragment reads are bank-conflict free.  A [M x K] is K-contiguous.  The
// right operand is W [K x N] (N-contiguous; fragments come from the LDS
// transpose read ds_read_b64_tr_b16) or K [N x K] (K-contiguous).
//
// The MFMA is issued with its operands swapped (MFMA A = right operand,
// MFMA B = left operand) and a fixed permutation of the right operand's
// columns, so each lane's 16 accumulator values are 16 CONSECUTIVE columns of
// ONE output row: row statistics are mostly thread-local.
//
// Epilogue ([ComFuse] Fig. 3 stage chain with bypass; inter-CTA level with
// dual-mode aggregation): the accumulator stays in registers through every
// stage.  The residual tile arrives through LDS with coalesced loads; per-row
// statistics reduce thread -> lane pair -> LDS (across column waves) -> across
// the tiles of the row group through global memory with an in-kernel join.
// Small row groups aggregate peer to peer (every member reads every partial);
// large ones elect the last arriver as leader, which combines and publishes
// one result per row that followers read, keeping the exchange traffic linear
// in the group size.  The output tile is staged in LDS and written as whole
// rows.  A persistent grid walks tiles in rounds of whole row groups sized to
// what is resident at once ([AStitch] "What it costs"); each output element
// has one owner ([sass2mlir] "Epilogue fusion").
#include <utility>

#include "dev.hpp"
#include "kernels.hpp"

namespace cf {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) f32x4 lds_f32x4_t;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;

constexpr int kThreads = 256;
constexpr uint32_t kOOB = 0x80000000u;  // buffer offset beyond every range: reads zero

// 16-byte-chunk XOR swizzles for K-contiguous tiles [rows][BK].  LDS has 64
// banks of 4 bytes (256 bytes); a 16-byte fragment read is served 16 lanes at
// a time, so the 16 rows one lane group reads at one logical chunk must land
// in 16 distinct 16-byte bank slots.  A row of 2*BK bytes shares its slots
// with the rows RPB = 256/(2*BK) apart, so the XOR takes the row bits above
// log2(RPB) (measured on MI355X with SQ_LDS_BANK_CONFLICT: the earlier
// row % 8 swizzle cost 3.9 stall cycles per 16-byte read, these none).
// Rows read in order (lanes 0..15 = 16 consecutive rows):
template <int BK>
__device__ __forceinline__ int swz(int row, int c) {
  static_assert(BK == 32 || BK == 64 || BK == 128, "swizzled depth");
  constexpr int CPR = BK / 8, RPB = 128 / BK;
  return c ^ ((row / RPB) % CPR);
}
// Rows read through the sigma permutation (lanes 0..15 = rows 0-3, 16-19,
// 4-7, 20-23 of a 32-row block): the varying row bits are 0, 1, 2 and 4.
template <int BK>
__device__ __forceinline__ int swz_sigma(int row, int c) {
  static_assert(BK == 32 || BK == 64 || BK == 128, "swizzled depth");
  constexpr int CPR = BK / 8, RPB = 128 / BK;
  return c ^ (((row / RPB) & (CPR / 2 - 1)) | (((row >> 4) & 1) * (CPR / 2)));
}

// Byte-offset XOR for N-contiguous tiles [BK][BN] read with the transpose
// read: the 4 k-rows one read touches land 64 bytes apart modulo the bank
// width, so their 64-byte segments cover all banks once (rows >= 256 bytes).
__device__ __forceinline__ int nn_mask(int k) { return (k & 3) << 6; }

// Output column (within a 32-column block) of MFMA row i under the permutation
// that gives lane l the columns 16*(l>>5) .. 16*(l>>5)+15.
__device__ __forceinline__ int sigma(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

// 16-byte chunk swizzle of the epilogue's row-major LDS tiles (residual in,
// output out; rows of >= 256 bytes): lanes 0..31 touch 32 rows at one column.
__device__ __forceinline__ int eswz(int row, int c) { return c ^ (row & 15); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// One 16-byte direct global->LDS load per lane: lane p of the wave writes
// lds_base + 16 * p (lds_base is wave-uniform).  voff = kOOB loads zeros.
__device__ __forceinline__ void g2l16(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_base, 16, (int)voff, 0, 0, 0);
}

template <int BM, int BN, int BK, bool NN, int NWAVES = 4>
struct Ring {
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int B_BYTES = BN * BK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LA = A_BYTES / (NWAVES * 1024);  // 1 KB wave loads per thread for A
  static constexpr int LB = B_BYTES / (NWAVES * 1024);
  static_assert(LA * NWAVES * 1024 == A_BYTES && LB * NWAVES * 1024 == B_BYTES, "tile bytes per workgroup load");
  static_assert(!NN || BN * 2 >= 256, "transpose-read swizzle needs rows of at least 256 bytes");

  // Lane p of wave w in load j writes LDS byte (j*NWAVES + w)*1024 + 16p of
  // the operand region and fetches the global chunk that belongs at that
  // (swizzled) position.  Its global byte offset is a uniform part (tile
  // origin and k0) plus a per-lane part fixed for the whole kernel, kept in
  // ao / bo.  Rows past M (A), past N (K) and W's rows past K fall outside the
  // buffer's range and read zero.  A chunk of W past N wraps into the next
  // row but feeds only output columns past N, which are never stored or
  // counted.  A chunk past K of a K-contiguous operand (A, K) would wrap into
  // the next row, so the last k-stage masks those to zero.
  uint32_t ao[LA], bo[LB];
  int N, K;

  __device__ __forceinline__ explicit Ring(const GemmArgs& a) : N((int)a.N), K((int)a.K) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < LA; ++j) {
      const int o = (j * NWAVES + w) * 1024 + lane * 16;
      const int row = o / (BK * 2), c = swz<BK>(row, (o % (BK * 2)) / 16);
      ao[j] = (uint32_t)(row * K + 8 * c) * 2u;
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      const int o = (j * NWAVES + w) * 1024 + lane * 16;
      if constexpr (NN) {
        const int k = o / (BN * 2), cb = ((o % (BN * 2)) ^ nn_mask(k)) / 16;
        bo[j] = (uint32_t)(k * N + 8 * cb) * 2u;
      } else {
        const int row = o / (BK * 2), c = swz_sigma<BK>(row, (o % (BK * 2)) / 16);
        bo[j] = (uint32_t)(row * K + 8 * c) * 2u;
      }
    }
  }

  // Issue the direct loads of one K-stage into `st`.
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, char* st, int m0,
                                       int n0, int k0) const {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const bool ktail = k0 + BK > K;
    const uint32_t ab = (uint32_t)(m0 * K + k0) * 2u;
    const uint32_t bb = NN ? (uint32_t)(k0 * N + n0) * 2u : (uint32_t)(n0 * K + k0) * 2u;
#pragma unroll
    for (int j = 0; j < LA; ++j) {
      uint32_t off = ab + ao[j];
      if (ktail) {
        const int o = (j * NWAVES + w) * 1024 + lane * 16;
        const int c = swz<BK>(o / (BK * 2), (o % (BK * 2)) / 16);
        if (k0 + 8 * c >= K) off = kOOB;
      }
      g2l16(ra, st + (j * NWAVES + w) * 1024, off);
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      uint32_t off = bb + bo[j];
      if (!NN && ktail) {
        const int o = (j * NWAVES + w) * 1024 + lane * 16;
        const int c = swz_sigma<BK>(o / (BK * 2), (o % (BK * 2)) / 16);
        if (k0 + 8 * c >= K) off = kOOB;
      }
      g2l16(rb, st + A_BYTES + (j * NWAVES + w) * 1024, off);
    }
  }
};

// Fragment reads for one 16-deep k-step from an LDS stage.
template <int BM, int BN, int BK, bool NN, int RB, int CB>
__device__ __forceinline__ void load_frags(const char* st, int ks, bf16x8_t (&bop)[RB], bf16x8_t (&aop)[CB], int wm,
                                           int wn) {
  constexpr int WM = RB * 32, WN = CB * 32;
  const int lane = threadIdx.x & 63;
  const uint16_t* As = reinterpret_cast<const uint16_t*>(st);
  const char* Bs = st + BM * BK * 2;
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
        const char* p = Bs + k * (BN * 2) + ((2 * n) ^ nn_mask(k));
        h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
      }
      aop[cb] = __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
      const int n = wn * WN + cb * 32 + sigma(lane & 31);
      const int c = 2 * ks + (lane >> 5);
      aop[cb] = *reinterpret_cast<const bf16x8_t*>(reinterpret_cast<const uint16_t*>(Bs) + n * BK +
                                                   8 * swz_sigma<BK>(n, c));
    }
  }
}

// One BK-deep stage of MFMAs from LDS.  The fragments of k-step ks+1 are all
// read before the MFMAs of step ks issue (two fragment register sets), with
// hard scheduling barriers around each group: otherwise the compiler pulls
// each read down next to its MFMA and reuses one register set, and every
// MFMA then waits out a full LDS latency.
template <int BM, int BN, int BK, bool NN, int RB, int CB, int NVMEM>
__device__ __forceinline__ void mma_stage(const char* st, f32x16 (&acc)[RB][CB], int wm, int wn) {
  constexpr int KS = BK / 16;
  bf16x8_t bop[2][RB], aop[2][CB];
  load_frags<BM, BN, BK, NN, RB, CB>(st, 0, bop[0], aop[0], wm, wn);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < KS) load_frags<BM, BN, BK, NN, RB, CB>(st, ks + 1, bop[cur ^ 1], aop[cur ^ 1], wm, wn);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[cur][cb], bop[cur][rb], acc[rb][cb], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Cross-wave (column waves) combine of per-row values through LDS.
// red: 2 slots x WGN x BM floats; the slot alternates per call, so one barrier
// per reduction suffices.
template <class Op, int BM, int WGN, int RB>
__device__ __forceinline__ void tile_row_reduce(float (&v)[RB], float* red, int& slot, int wm, int wn) {
  constexpr int WM = RB * 32;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) v[rb] = Op::op(v[rb], __shfl_xor(v[rb], 32, kWave));
  float* s = red + slot * (WGN * BM);
  if (lane < 32) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) s[wn * BM + wm * WM + rb * 32 + lane] = v[rb];
  }
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = wm * WM + rb * 32 + (lane & 31);
    float x = s[r];
#pragma unroll
    for (int q = 1; q < WGN; ++q) x = Op::op(x, s[q * BM + r]);
    v[rb] = x;
  }
  slot ^= 1;
}

// Row statistics merges (member order fixed, so every member gets identical bits).
// LN: (count, mean, M2) by Chan's pairwise update.  Softmax: (max, sum) online.
struct MergeLN {
  float n = 0.f, mean = 0.f, m2 = 0.f;
  __device__ void add(float4 q) {
    const float nb = q.x;
    if (nb == 0.f) return;
    const float nn = n + nb;
    const float d = q.y - mean;
    mean += d * (nb / nn);
    m2 += q.z + d * d * (n * nb / nn);
    n = nn;
  }
  __device__ float4 part() const { return make_float4(n, mean, m2, 0.f); }
};
struct MergeSM {
  float m = -INFINITY, l = 0.f;
  __device__ void add(float4 q) {
    if (q.x == -INFINITY) return;
    if (q.x > m) {
      l = l * __builtin_amdgcn_exp2f(m - q.x) + q.y;
      m = q.x;
    } else {
      l += q.y * __builtin_amdgcn_exp2f(q.x - m);
    }
  }
  __device__ float4 part() const { return make_float4(m, l, 0.f, 0.f); }
};

// MainLoop of one tile over a two-slot ring (slot objects s0, s1).  On entry
// stage 0 of the tile has been issued into s0.  Stage kt lives in slot kt & 1:
// each step waits for its own stage, publishes it with a barrier (which also
// retires the other slot), issues the next stage into the other slot and
// computes.  With `nxt`, stage 0 of the tile at (nm0, nn0) goes into s0 as
// soon as s0 is free, so its latency overlaps the caller's epilogue.  Waves
// may still read s1 on return; the next call's first barrier covers that.
template <int BM, int BN, int BK, bool NN, int RB, int CB, int NWAVES = 4>
__device__ __forceinline__ void main_loop(const Ring<BM, BN, BK, NN, NWAVES>& rg, __amdgpu_buffer_rsrc_t rA,
                                          __amdgpu_buffer_rsrc_t rB,
                                          char* s0, char* s1, int m0, int n0, bool nxt, int nm0, int nn0,
                                          f32x16 (&acc)[RB][CB], int KT, int wm, int wn) {
  using RG = Ring<BM, BN, BK, NN, NWAVES>;
  constexpr int NV = RG::LA + RG::LB;
  for (int kt = 0; kt < KT; kt += 2) {
    wait_vm<0>();
    __syncthreads();
    const bool two = kt + 1 < KT;
    if (two) rg.load(rA, rB, s1, m0, n0, (kt + 1) * BK);
    mma_stage<BM, BN, BK, NN, RB, CB, NV>(s0, acc, wm, wn);
    if (!two) {
      if (nxt) {
        __syncthreads();  // every wave is done with s0
        rg.load(rA, rB, s0, nm0, nn0, 0);
      }
      break;
    }
    wait_vm<0>();
    __syncthreads();
    if (kt + 2 < KT) rg.load(rA, rB, s0, m0, n0, (kt + 2) * BK);
    else if (nxt) rg.load(rA, rB, s0, nm0, nn0, 0);
    mma_stage<BM, BN, BK, NN, RB, CB, NV>(s1, acc, wm, wn);
  }
}

// s_waitcnt vmcnt(n) for a run-time n in [0, 63] (one immediate per case).
__device__ __forceinline__ void wait_vm_n(int n) {
  switch (n) {
#define CF_W(k) \
  case k:       \
    wait_vm<k>(); \
    return;
    CF_W(0) CF_W(1) CF_W(2) CF_W(3) CF_W(4) CF_W(5) CF_W(6) CF_W(7) CF_W(8) CF_W(9) CF_W(10) CF_W(11) CF_W(12)
    CF_W(13) CF_W(14) CF_W(15) CF_W(16) CF_W(17) CF_W(18) CF_W(19) CF_W(20) CF_W(21) CF_W(22) CF_W(23) CF_W(24)
    CF_W(25) CF_W(26) CF_W(27) CF_W(28) CF_W(29) CF_W(30) CF_W(31) CF_W(32)
#undef CF_W
    default:
      wait_vm<32>();
      return;
  }
}

// MainLoop of one tile over an NS-slot ring (separate LDS objects sl[0..NS-1],
// so the compiler can tell the slot being read from the ones being filled).
// Stage s lives in slot s % NS and is issued NS-1 stages ahead, so NS-1 loads
// are in flight behind the one being computed; each step waits only for its
// own stage (vector-memory loads complete in issue order), publishes it with
// a barrier that also retires the slot computed last, refills that slot and
// computes.  On entry stages 0 .. min(NS-1, KT)-1 of the tile have been issued
// into slots 0, 1, ...  With `nxt` (requires KT % NS == 0), stages 0 .. NS-2
// of the tile at (nm0, nn0) are issued the same way as the tail frees slots,
// so the next call's entry condition holds and their latency overlaps the
// caller's epilogue.
// `on_stage(st)` runs after stage st's barrier and ring refill, before its
// MFMAs (an epilogue can issue its first loads behind the last stages).
struct NoStageHook {
  __device__ void operator()(int) const {}
};
template <int BM, int BN, int BK, bool NN, int RB, int CB, int NWAVES, int NS, class Hook = NoStageHook>
__device__ __forceinline__ void main_loop_ns(const Ring<BM, BN, BK, NN, NWAVES>& rg, __amdgpu_buffer_rsrc_t rA,
                                             __amdgpu_buffer_rsrc_t rB, char* const (&sl)[NS], int m0, int n0,
                                             bool nxt, int nm0, int nn0, f32x16 (&acc)[RB][CB], int KT, int wm,
                                             int wn, Hook on_stage = Hook{}) {
  using RG = Ring<BM, BN, BK, NN, NWAVES>;
  constexpr int LPS = RG::LA + RG::LB;  // loads per lane per stage
  static_assert(NS >= 2 && (NS - 2) * LPS <= 32, "ring depth");
  for (int kt = 0; kt < KT; kt += NS) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int st = kt + i;
      if (st >= KT) break;
      // stages issued after this one, whose loads may stay in flight
      const int after = nxt ? NS - 2 : min(NS - 2, KT - 1 - st);
      wait_vm_n(after * LPS);
      __syncthreads();
      const int sn = st + NS - 1;
      if (sn < KT) rg.load(rA, rB, sl[(i + NS - 1) % NS], m0, n0, sn * BK);
      else if (nxt && sn - KT < NS - 1) rg.load(rA, rB, sl[(i + NS - 1) % NS], nm0, nn0, (sn - KT) * BK);
      on_stage(st);
      mma_stage<BM, BN, BK, NN, RB, CB, LPS>(sl[i], acc, wm, wn);
    }
  }
}

// Issue the first min(NS-1, KT) stages of a tile into slots 0, 1, ...
template <int BM, int BN, int BK, bool NN, int NWAVES, int NS>
__device__ __forceinline__ void prologue_ns(const Ring<BM, BN, BK, NN, NWAVES>& rg, __amdgpu_buffer_rsrc_t rA,
                                            __amdgpu_buffer_rsrc_t rB, char* const (&sl)[NS], int m0, int n0,
                                            int KT) {
#pragma unroll
  for (int q = 0; q < NS - 1; ++q)
    if (q < KT) rg.load(rA, rB, sl[q], m0, n0, q * BK);
}

// Pairwise merges of row statistics.  Both are symmetric in their arguments
// up to the order fixed by the caller, so lanes that merge the same values in
// the same order hold identical bits.
// Softmax (max, sum of 2^(s - max)) in the base-2 domain.
__device__ __forceinline__ void merge_sm(float& m, float& l, float mo, float lo) {
  const float mx = fmaxf(m, mo);
  if (mx == -INFINITY) {
    m = mx;
    l = 0.0f;
    return;
  }
  l = l * __builtin_amdgcn_exp2f(m - mx) + lo * __builtin_amdgcn_exp2f(mo - mx);
  m = mx;
}
// LayerNorm (count, mean, M2): Chan's pairwise update, (a) then (b).
__device__ __forceinline__ void merge_ln(float& n, float& mu, float& m2, float nb, float mub, float m2b) {
  if (nb == 0.0f) return;
  if (n == 0.0f) {
    n = nb;
    mu = mub;
    m2 = m2b;
    return;
  }
  const float nn = n + nb, d = mub - mu;
  mu += d * (nb / nn);
  m2 += m2b + d * d * (n * nb / nn);
  n = nn;
}

// Tile-level row statistics from per-lane ones: the lane pair that shares a
// row (lanes l and l ^ 32) merges lower half first, then the WGN column waves
// merge through LDS in wave order.  Every lane of the row ends with the same
// bits.  One barrier; `red` must not be rewritten before the next barrier.
template <int BM, int WGN, int RB>
__device__ __forceinline__ void tile_merge_sm(float (&m)[RB], float (&l)[RB], float2* red, int wm, int wn) {
  constexpr int WM = RB * 32;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float mo = __shfl_xor(m[rb], 32, kWave), lo = __shfl_xor(l[rb], 32, kWave);
    merge_sm(m[rb], l[rb], mo, lo);
    if (lane < 32) red[wn * BM + wm * WM + rb * 32 + lane] = make_float2(m[rb], l[rb]);
  }
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = wm * WM + rb * 32 + (lane & 31);
    float2 x = red[r];
#pragma unroll
    for (int q = 1; q < WGN; ++q) merge_sm(x.x, x.y, red[q * BM + r].x, red[q * BM + r].y);
    m[rb] = x.x;
    l[rb] = x.y;
  }
}
template <int BM, int WGN, int RB>
__device__ __forceinline__ void tile_merge_ln(float (&n)[RB], float (&mu)[RB], float (&m2)[RB], float4* red, int wm,
                                              int wn) {
  constexpr int WM = RB * 32;
  const int lane = threadIdx.x & 63;
  const bool lo_half = lane < 32;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float no = __shfl_xor(n[rb], 32, kWave), muo = __shfl_xor(mu[rb], 32, kWave),
                m2o = __shfl_xor(m2[rb], 32, kWave);
    if (lo_half) {
      merge_ln(n[rb], mu[rb], m2[rb], no, muo, m2o);
    } else {
      float a0 = no, a1 = muo, a2 = m2o;
      merge_ln(a0, a1, a2, n[rb], mu[rb], m2[rb]);
      n[rb] = a0;
      mu[rb] = a1;
      m2[rb] = a2;
    }
    if (lo_half) red[wn * BM + wm * WM + rb * 32 + lane] = make_float4(n[rb], mu[rb], m2[rb], 0.0f);
  }
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = wm * WM + rb * 32 + (lane & 31);
    float4 x = red[r];
#pragma unroll
    for (int q = 1; q < WGN; ++q) merge_ln(x.x, x.y, x.z, red[q * BM + r].x, red[q * BM + r].y, red[q * BM + r].z);
    n[rb] = x.x;
    mu[rb] = x.y;
    m2[rb] = x.z;
  }
}

// Spin until the join word's generation differs from gen0 (one lane).  The
// poll interval is ~0.2 us: hundreds of waiting workgroups polling a few join
// words back to back slow down the device-scope loads of the workgroups they
// wait for.
__device__ __forceinline__ void wait_generation(uint64_t* jw, uint32_t gen0, uint32_t* err) {
  uint32_t it = 0;
  for (; it < kSpinCap; ++it) {
    const uint64_t wv = __hip_atomic_load(jw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(wv >> 32) != gen0) break;
    __builtin_amdgcn_s_sleep(8);
  }
  if (it == kSpinCap) __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int EPI, int BM, int BN, int BK, int STAGES>
constexpr int gemm_lds_bytes() {
  constexpr int ring = (BM + BN) * BK * 2;  // slot 0 (slot 1 is its own object)
  // bf16 tile + red (2 x 4 x BM floats) + pub (BM float4) + parts (256 float4) + stat (BM float2) + flags
  constexpr int epi = EPI == kEpiStoreF32 ? BM * BN * 4 / 4
                      : EPI == kEpiAct    ? BM * BN * 2 + BN * 4  // bf16 tile + bias slice
                                          : BM * BN * 2 + 32 * BM + 16 * BM + 16 * 256 + 8 * BM + 64 + 3 * BN * 4;
  return ring > epi ? ring : epi;
}

template <int V>
struct IntC {
  static constexpr int value = V;
};
// f(IntC<Q>{}) for Q = 0, 1, ..., in order
template <class F, int... Q>
__device__ __forceinline__ void for_each_c(F&& f, std::integer_sequence<int, Q...>) {
  (f(IntC<Q>{}), ...);
}

// Unary activations of the activation epilogue, in fp32.  Both sigmoid-gated
// forms use 1 / (1 + 2^t): the tanh-form GELU 0.5 u (1 + tanh z), with
// z = sqrt(2/pi) (u + 0.044715 u^3), equals u * sigmoid(2 z) because
// 1 + tanh z = 2 / (1 + e^(-2z)); SiLU is u * sigmoid(u).  For t past the
// exp2 range the gate is 1 / inf = 0 (or 1 / 1 = 1), the exact limits.
constexpr float kGeluT1 = -2.302208198144325f;    // -2 sqrt(2/pi) log2(e)
constexpr float kGeluT3 = -0.1029432395800235f;   // the same times 0.044715
template <int ACT>
__device__ __forceinline__ float act_fn(float u) {
  if constexpr (ACT == kActRelu) {
    return fmaxf(u, 0.0f);
  } else if constexpr (ACT == kActGeluTanh) {
    const float t = u * fmaf(kGeluT3, u * u, kGeluT1);
    return u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
  } else if constexpr (ACT == kActSilu) {
    return u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * u));
  } else if constexpr (ACT == kActSquare) {
    return u * u;
  } else if constexpr (ACT == kActRsqrt) {
    return __builtin_amdgcn_rsqf(u);
  } else {
    return u;
  }
}

}  // namespace

template <int EPI, bool NN, int BM, int BN, int BK, int WGM, int STAGES, int MINB>
__global__ __launch_bounds__(kThreads, MINB) void k_gemm(GemmArgs a) {
  using RG = Ring<BM, BN, BK, NN>;
  constexpr int WGN = 4 / WGM;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int RB = WM / 32, CB = WN / 32;
  constexpr int LDS = gemm_lds_bytes<EPI, BM, BN, BK, STAGES>();
  constexpr int C16 = BN * 2 / 16;  // 16-byte chunks per bf16 output row
  static_assert(STAGES == 2, "ring slots are separate LDS objects; two are instantiated");
  constexpr int NP = BM >= kThreads ? 1 : kThreads / BM;  // threads combining one row's partials
  static_assert(WM % 32 == 0 && WN % 32 == 0 && WGM * WGN == 4, "wave tile");
  static_assert(C16 >= 16 && (BM * C16) % kThreads == 0, "epilogue tile");
  // Ring slot 0 doubles as the epilogue's LDS; slot 1 is a separate object so
  // the compiler can see that fragment reads of one slot never alias the
  // direct loads filling the other (no conservative wait on the prefetch).
  __shared__ __align__(16) char lds[LDS];
  __shared__ __align__(16) char lds1[RG::STAGE_BYTES];

  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int wm = w / WGN, wn = w % WGN;
  const int hl = lane >> 5, l32 = lane & 31;
  const int KT = (int)((a.K + BK - 1) / BK);
  const uint32_t G = gridDim.x;
  const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
  const uint32_t g = (EPI == kEpiStoreF32) ? blockIdx.x : xcd_local_id(blockIdx.x, G);
  const __amdgpu_buffer_rsrc_t rA = rsrc(a.A, (uint32_t)(a.M * a.K * 2));
  const __amdgpu_buffer_rsrc_t rB = rsrc(a.B, (uint32_t)(a.N * a.K * 2));
  const RG rg(a);

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
    rg.load(rA, rB, lds, (int)m0, (int)n0, 0);
    main_loop<BM, BN, BK, NN, RB, CB>(rg, rA, rB, lds, lds1, (int)m0, (int)n0, false, 0, 0, acc, KT, wm, wn);
    wait_vm<0>();
    __syncthreads();  // every wave is done with the ring: it is free from here on

    // lane's output coordinates: row(rb) = m0 + wm*WM + rb*32 + l32,
    // cols(cb) = n0 + wn*WN + cb*32 + 16*hl + [0, 16)
    if constexpr (EPI == kEpiStoreF32) {
      // fp32 tile staged through LDS a quarter tile at a time, written as rows
      float* ot = reinterpret_cast<float*>(lds);
      constexpr int F4 = BN / 4;     // float4 chunks per row
      constexpr int QROWS = BM / 4;  // rows per quarter
      for (int qt = 0; qt < 4; ++qt) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int rl = wm * WM + rb * 32 + l32;
          if (rl / QROWS != qt) continue;
          const int rr = rl - qt * QROWS;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            const int c4 = (wn * WN + cb * 32 + 16 * hl) / 4;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<float4*>(ot + rr * BN + 4 * ((c4 + q) ^ (rr & 15))) =
                  make_float4(acc[rb][cb][4 * q], acc[rb][cb][4 * q + 1], acc[rb][cb][4 * q + 2],
                              acc[rb][cb][4 * q + 3]);
          }
        }
        __syncthreads();
        for (int id = t; id < QROWS * F4; id += kThreads) {
          const int rr = id / F4, c = id % F4;
          const int64_t row = m0 + qt * QROWS + rr, col = n0 + 4 * c;
          if (row < a.M && col < a.N)
            st4_stream(a.Z + row * a.N + col, *reinterpret_cast<const float4*>(ot + rr * BN + 4 * (c ^ (rr & 15))));
        }
        __syncthreads();
      }
    } else if constexpr (EPI == kEpiAct) {
      // y = act(acc + bias_j) per element: no cross-tile dependency.  The bias
      // slice goes to LDS (zero past N or without bias), the bf16 results to
      // the LDS output tile, then whole row segments out.
      uint16_t* tile16 = reinterpret_cast<uint16_t*>(lds);
      float* vec = reinterpret_cast<float*>(lds + BM * BN * 2);
      for (int id = t; id < BN / 4; id += kThreads) {
        const int64_t gn = n0 + 4 * id;
        reinterpret_cast<float4*>(vec)[id] = (a.bias != nullptr && gn < a.N)
                                                 ? *reinterpret_cast<const float4*>(a.bias + gn)
                                                 : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      __syncthreads();
      auto finish = [&](auto actc) {
        constexpr int ACT = decltype(actc)::value;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int cl0 = wn * WN + cb * 32 + 16 * hl;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float4 b0 = *reinterpret_cast<const float4*>(vec + cl0 + 8 * h);
            const float4 b1 = *reinterpret_cast<const float4*>(vec + cl0 + 8 * h + 4);
            const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
              const int rl = wm * WM + rb * 32 + l32;
              float o[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) o[e] = act_fn<ACT>(acc[rb][cb][8 * h + e] + bb[e]);
              const u32x4 pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                                pack_bf16x2(o[6], o[7])};
              *reinterpret_cast<u32x4*>(tile16 + rl * BN + 8 * eswz(rl, cl0 / 8 + h)) = pk;
            }
          }
        }
      };
      switch (a.act) {
        case kActRelu: finish(IntC<kActRelu>{}); break;
        case kActGeluTanh: finish(IntC<kActGeluTanh>{}); break;
        case kActSilu: finish(IntC<kActSilu>{}); break;
        case kActSquare: finish(IntC<kActSquare>{}); break;
        case kActRsqrt: finish(IntC<kActRsqrt>{}); break;
        default: finish(IntC<kActNone>{}); break;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < BM * C16 / kThreads; ++j) {
        const int id = j * kThreads + t;
        const int rr = id / C16, c = id % C16;
        const int64_t row = m0 + rr, col = n0 + 8 * c;
        if (row < a.M && col < a.N)
          __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(tile16 + rr * BN + 8 * eswz(rr, c)),
                                      reinterpret_cast<u32x4*>(a.Y + row * a.N + col));
      }
    } else {
      // LDS carve-up (the ring is free): output / residual tile, then scratch.
      uint16_t* tile16 = reinterpret_cast<uint16_t*>(lds);                  // BM x BN bf16
      float* red = reinterpret_cast<float*>(lds + BM * BN * 2);              // 2 x WGN x BM
      float4* pub = reinterpret_cast<float4*>(red + 2 * 4 * BM);             // BM
      float4* parts = pub + BM;                                              // 256 (NP per row)
      float2* stat = reinterpret_cast<float2*>(parts + kThreads);            // BM
      int* flag = reinterpret_cast<int*>(stat + BM);                         // last-arriver flag, gen0
      float* vec = reinterpret_cast<float*>(flag + 16);                      // bias | gamma | beta slices (BN each)
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
        // residual tile -> LDS with coalesced direct loads (whole rows)
        if (a.R != nullptr) {
          const __amdgpu_buffer_rsrc_t rR = rsrc(a.R, (uint32_t)(a.M * a.N * 2));
#pragma unroll
          for (int j = 0; j < BM * C16 / kThreads; ++j) {
            const int o = (j * 4 + w) * 1024 + lane * 16;
            const int row = o / (BN * 2), pc = (o % (BN * 2)) / 16;
            const int c = eswz(row, pc);
            const int64_t gm = m0 + row, gn = n0 + 8 * c;
            const uint32_t off = (gm < a.M && gn < a.N) ? (uint32_t)((gm * a.N + gn) * 2) : kOOB;
            g2l16(rR, lds + (j * 4 + w) * 1024, off);
          }
        }
        // bias / gamma / beta slices of this tile -> LDS (zero past N), so the
        // epilogue reads them from LDS instead of holding them in registers
        {
          constexpr int V4 = BN / 4;  // float4 chunks per slice
          for (int id = t; id < 3 * V4; id += kThreads) {
            const int which = id / V4, c = id % V4;
            const int64_t gn = n0 + 4 * c;
            const float* src = which == 0 ? a.bias : (which == 1 ? a.gamma : a.beta);
            reinterpret_cast<float4*>(vec + which * BN)[c] =
                gn < a.N ? *reinterpret_cast<const float4*>(src + gn) : make_float4(0.f, 0.f, 0.f, 0.f);
          }
        }
        wait_vm<0>();
        __syncthreads();
        // stage 1: u = acc + bias_j + R_ij, kept in the accumulator registers
        // (one column block at a time, so only its 16 bias values are live)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int cl0 = wn * WN + cb * 32 + 16 * hl;
          float bv[16];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 b = *reinterpret_cast<const float4*>(vec + cl0 + 4 * q);
            bv[4 * q] = b.x; bv[4 * q + 1] = b.y; bv[4 * q + 2] = b.z; bv[4 * q + 3] = b.w;
          }
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const int rl = wm * WM + rb * 32 + l32;
            u32x4 rr[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
            if (a.R != nullptr) {
#pragma unroll
              for (int h = 0; h < 2; ++h)
                rr[h] = *reinterpret_cast<const u32x4*>(tile16 + rl * BN + 8 * eswz(rl, cl0 / 8 + h));
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const uint32_t wv = rr[r >> 3][(r & 7) >> 1];
              const float u = acc[rb][cb][r] + bv[r] + ((r & 1) ? bf16_hi(wv) : bf16_lo(wv));
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
        tile_row_reduce<OpSum, BM, WGN, RB>(s, red, slot, wm, wn);
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
        tile_row_reduce<OpSum, BM, WGN, RB>(s, red, slot, wm, wn);
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
        tile_row_reduce<OpMax, BM, WGN, RB>(mx, red, slot, wm, wn);
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
        tile_row_reduce<OpSum, BM, WGN, RB>(l, red, slot, wm, wn);
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
      uint64_t* jw = a.joins + g / a.tiles_n;  // the members of a row group share g / tiles_n every round
      const int T = a.tiles_n;
      if (w == 0) {
        float4* P = reinterpret_cast<float4*>(a.partials);
        for (int r = lane; r < BM; r += kWave) {
          const int64_t row = m0 + r;
          if (row < a.M) st_dev4(P + (size_t)row * T + tn, pub[r]);
        }
        wait_stores();
        if (lane == 0) {
          const uint64_t old = __hip_atomic_fetch_add(jw, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          flag[0] = ((uint32_t)old == (uint32_t)(T - 1)) ? 1 : 0;
          flag[1] = (int)(uint32_t)(old >> 32);
        }
      }
      __syncthreads();
      const bool last = flag[0] != 0;
      const uint32_t gen0 = (uint32_t)flag[1];
      const bool leader_mode = a.agg_leader != 0;

      // Combine every row's T partials with all 256 threads: thread t merges
      // part t / BM (a contiguous run of members) of row t % BM, then one
      // thread per row merges the NP parts in order.  Device-scope loads.
      auto combine_rows = [&]() {
        const int r = t % BM, q = t / BM;
        const int per = (T + NP - 1) / NP;
        const int kb = q * per, ke = min(T, kb + per);
        const float4* P = reinterpret_cast<const float4*>(a.partials) + (size_t)(m0 + r) * T;
        const bool valid = (m0 + r < a.M) && q < NP;
        float4 part;
        if constexpr (EPI == kEpiLN) {
          MergeLN mg;
          if (valid)
            for (int k0 = kb; k0 < ke; k0 += 8) {
              float4 v[8];
#pragma unroll
              for (int k = 0; k < 8; ++k) v[k] = k0 + k < ke ? ld_dev4(P + k0 + k) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
              for (int k = 0; k < 8; ++k) mg.add(v[k]);
            }
          part = mg.part();
        } else {
          MergeSM mg;
          if (valid)
            for (int k0 = kb; k0 < ke; k0 += 8) {
              float4 v[8];
#pragma unroll
              for (int k = 0; k < 8; ++k)
                v[k] = k0 + k < ke ? ld_dev4(P + k0 + k) : make_float4(-INFINITY, 0.f, 0.f, 0.f);
#pragma unroll
              for (int k = 0; k < 8; ++k) mg.add(v[k]);
            }
          part = mg.part();
        }
        if (q < NP) parts[q * BM + r] = part;
        __syncthreads();
        if (t < BM) {
          float2 st2 = make_float2(0.f, 0.f);
          if (m0 + t < a.M) {
            if constexpr (EPI == kEpiLN) {
              MergeLN mg;
              for (int k = 0; k < NP; ++k) mg.add(parts[k * BM + t]);
              st2 = make_float2(mg.mean, rsqrtf(mg.m2 / (float)a.N + a.eps));
            } else {
              MergeSM mg;
              for (int k = 0; k < NP; ++k) mg.add(parts[k * BM + t]);
              st2 = make_float2(mg.m, 1.0f / mg.l);
            }
          }
          stat[t] = st2;
        }
      };
      auto wait_gen = [&]() {
        uint32_t it = 0;
        for (; it < kSpinCap; ++it) {
          const uint64_t wv = __hip_atomic_load(jw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((uint32_t)(wv >> 32) != gen0) break;
          __builtin_amdgcn_s_sleep(1);
        }
        if (it == kSpinCap) __hip_atomic_fetch_or(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      };

      float2* fin = reinterpret_cast<float2*>(a.finals);
      if (leader_mode) {
        if (last) {
          // leader: combine every row of the group once, publish, release
          combine_rows();
          if (t < BM && m0 + t < a.M) {
            st_dev(reinterpret_cast<float*>(fin + m0 + t), stat[t].x);
            st_dev(reinterpret_cast<float*>(fin + m0 + t) + 1, stat[t].y);
          }
          wait_stores();
          __syncthreads();
          if (t == 0) __hip_atomic_fetch_add(jw, (1ull << 32) - (uint64_t)T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          if (t == 0) wait_gen();
          __syncthreads();
          if (t < BM) {
            const int64_t row = m0 + t;
            stat[t] = row < a.M ? make_float2(ld_dev(reinterpret_cast<const float*>(fin + row)),
                                              ld_dev(reinterpret_cast<const float*>(fin + row) + 1))
                                : make_float2(0.f, 0.f);
          }
        }
      } else {
        // peer to peer: the last arriver releases at once; every member combines
        if (t == 0) {
          if (last) __hip_atomic_fetch_add(jw, (1ull << 32) - (uint64_t)T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          else wait_gen();
        }
        __syncthreads();
        combine_rows();
      }
      __syncthreads();

      // ------------------------------------------------ final stage + commit
      // results go to the LDS output tile (bf16, swizzled chunks), then rows out
      float fa[RB], fb[RB];  // LN: y = (acc - fb) * fa * gamma + beta; softmax: y = acc * fa
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float2 st2 = stat[wm * WM + rb * 32 + l32];
        if constexpr (EPI == kEpiLN) {
          fa[rb] = st2.y;
          fb[rb] = st2.x;
        } else {
          fa[rb] = __builtin_amdgcn_exp2f(p0[rb] - st2.x) * st2.y;
          fb[rb] = 0.f;
        }
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int cl0 = wn * WN + cb * 32 + 16 * hl;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float gg[8], bb[8];
          if constexpr (EPI == kEpiLN) {
            const float4 g0 = *reinterpret_cast<const float4*>(vec + BN + cl0 + 8 * h);
            const float4 g1 = *reinterpret_cast<const float4*>(vec + BN + cl0 + 8 * h + 4);
            const float4 b0 = *reinterpret_cast<const float4*>(vec + 2 * BN + cl0 + 8 * h);
            const float4 b1 = *reinterpret_cast<const float4*>(vec + 2 * BN + cl0 + 8 * h + 4);
            gg[0] = g0.x; gg[1] = g0.y; gg[2] = g0.z; gg[3] = g0.w; gg[4] = g1.x; gg[5] = g1.y; gg[6] = g1.z; gg[7] = g1.w;
            bb[0] = b0.x; bb[1] = b0.y; bb[2] = b0.z; bb[3] = b0.w; bb[4] = b1.x; bb[5] = b1.y; bb[6] = b1.z; bb[7] = b1.w;
          }
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const int rl = wm * WM + rb * 32 + l32;
            float o[8];
            if constexpr (EPI == kEpiLN) {
#pragma unroll
              for (int e = 0; e < 8; ++e) o[e] = fmaf((acc[rb][cb][8 * h + e] - fb[rb]) * fa[rb], gg[e], bb[e]);
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) o[e] = acc[rb][cb][8 * h + e] * fa[rb];
            }
            const u32x4 pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                              pack_bf16x2(o[6], o[7])};
            *reinterpret_cast<u32x4*>(tile16 + rl * BN + 8 * eswz(rl, cl0 / 8 + h)) = pk;
          }
        }
      }
      __syncthreads();
      // each wave instruction stores 1 KB of whole output row segments
#pragma unroll
      for (int j = 0; j < BM * C16 / kThreads; ++j) {
        const int id = j * kThreads + t;
        const int rr = id / C16, c = id % C16;
        const int64_t row = m0 + rr, col = n0 + 8 * c;
        if (row < a.M && col < a.N)
          __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(tile16 + rr * BN + 8 * eswz(rr, c)),
                                      reinterpret_cast<u32x4*>(a.Y + row * a.N + col));
      }
    }
    __syncthreads();  // LDS is reused by the next tile's prologue
  }
}

// ------------------------------------------- epilogues overlapped with MainLoops
//
// The round-based kernel above idles every member of a row group from its
// publish until the slowest member arrives.  The two kernels below keep the
// matrix cores busy across that wait instead.
//
// Lane (rb, cb) output coordinates, as above: row m0 + wm*WM + rb*32 + l32,
// 16 consecutive columns n0 + wn*WN + cb*32 + 16*hl + [0, 16).  With that
// layout each lane's 32 output bytes per (rb, cb) are contiguous, and the
// epilogues load and store them straight from registers (plain accesses, so
// the two 16-byte halves of a row segment written by different instructions
// merge in L2 before they reach HBM).


// 16-byte buffer accesses with 32-bit offsets (kOOB: loads read zero, stores
// are dropped).
__device__ __forceinline__ u32x4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ float4 bld16f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ void bst16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}

__device__ __forceinline__ float bld4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// The same with device-scope coherence (sc1), for cross-workgroup partials.
__device__ __forceinline__ u32x4 bld16_dev(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 16);
}
__device__ __forceinline__ void bst16_dev(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 16);
}

template <int RB, int CB>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[RB][CB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.0f;
}

// GEMM + row softmax in two sweeps over the same tile sequence.
//   Sweep 1: each tile's per-row (max, sum) in the base-2 domain is published
//   without waiting; the last member of a row block to arrive merges the
//   block's partials in member order and publishes (max, 1/sum) per row.
//   Sweep 2: each tile's product is computed again, scaled and normalised
//   with the merged statistics (waiting, rarely, for a block still in flight)
//   and stored as bf16.
// The product is recomputed rather than held across the wait: with a short
// reduction dimension the second MainLoop costs less than the exchange it
// hides, and the output tile never leaves registers.
template <int BM, int BN, int BK, int WGM, int MINB>
__global__ __launch_bounds__(kThreads, MINB) void k_gemm_sm2(GemmArgs a) {
  using RG = Ring<BM, BN, BK, false>;
  constexpr int WGN = 4 / WGM;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int RB = WM / 32, CB = WN / 32;
  constexpr int NP = kThreads / BM;  // threads merging one row's partials
  static_assert(BM <= kThreads && kThreads % BM == 0 && WM % 32 == 0 && WN % 32 == 0, "tile");
  __shared__ __align__(16) char s0[RG::STAGE_BYTES];
  __shared__ __align__(16) char s1[RG::STAGE_BYTES];
  __shared__ float2 red[WGN * BM];
  __shared__ float2 parts[kThreads];
  __shared__ uint32_t gens[kMaxRounds];
  __shared__ int last;

  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int wm = w / WGN, wn = w % WGN;
  const int hl = lane >> 5, l32 = lane & 31;
  const int lrow = wm * WM + l32, lcol = wn * WN + 16 * hl;  // lane's first row / column in a tile
  const int M = (int)a.M, N = (int)a.N;
  const int KT = (int)((a.K + BK - 1) / BK);
  const int G = (int)gridDim.x;
  const int g = (int)xcd_local_id(blockIdx.x, (uint32_t)G);
  const int T = a.tiles_n;
  const int tiles = a.tiles_m * T;
  if (g >= tiles) return;
  const __amdgpu_buffer_rsrc_t rA = rsrc(a.A, (uint32_t)(a.M * a.K * 2));
  const __amdgpu_buffer_rsrc_t rB = rsrc(a.B, (uint32_t)(a.N * a.K * 2));
  const __amdgpu_buffer_rsrc_t rY = rsrc(a.Y, (uint32_t)(a.M * a.N * 2));
  const float sc = a.scale * kLog2e;
  float2* P = reinterpret_cast<float2*>(a.partials);
  float2* F = reinterpret_cast<float2*>(a.finals);

  const RG rg(a);
  rg.load(rA, rB, s0, (g / T) * BM, (g % T) * BN, 0);

  // ------------------------------------------------ sweep 1: statistics
  int i = 0;
  for (int tile = g; tile < tiles; tile += G, ++i) {
    const int rowblk = tile / T, tn = tile - rowblk * T;
    const int m0 = rowblk * BM, n0 = tn * BN;
    const int nt = tile + G < tiles ? tile + G : g;  // sweep 2 starts again at g
    f32x16 acc[RB][CB];
    zero_acc(acc);
    main_loop<BM, BN, BK, false, RB, CB>(rg, rA, rB, s0, s1, m0, n0, true, (nt / T) * BM, (nt % T) * BN, acc, KT,
                                         wm, wn);
    float mr[RB], lr[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float m = -INFINITY;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (n0 + lcol + cb * 32 + (r & 8) < N) m = fmaxf(m, acc[rb][cb][r] * sc);
      float l = 0.0f;
      if (m != -INFINITY) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (n0 + lcol + cb * 32 + (r & 8) < N) l += __builtin_amdgcn_exp2f(acc[rb][cb][r] * sc - m);
      }
      mr[rb] = m;
      lr[rb] = l;
    }
    tile_merge_sm<BM, WGN, RB>(mr, lr, red, wm, wn);
    if (wn == 0 && hl == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int row = m0 + lrow + rb * 32;
        if (row < M) st_dev2(P + (size_t)row * T + tn, make_float2(mr[rb], lr[rb]));
      }
    }
    wait_stores();
    __syncthreads();
    uint64_t* jw = a.joins + rowblk;
    if (t == 0) {
      const uint64_t old = __hip_atomic_fetch_add(jw, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = ((uint32_t)old == (uint32_t)(T - 1)) ? 1 : 0;
      gens[i] = (uint32_t)(old >> 32);
    }
    __syncthreads();
    if (last) {
      // merge the block's rows: NP threads per row over contiguous runs of
      // members, then one thread per row over the NP runs, in order
      const int r = t % BM, q = t / BM;
      const int per = (T + NP - 1) / NP;
      const int kb = q * per, ke = min(T, kb + per);
      float m = -INFINITY, l = 0.0f;
      if (m0 + r < M) {
        const float2* Pr = P + (size_t)(m0 + r) * T;
        for (int k0 = kb; k0 < ke; k0 += 8) {
          float2 v[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) v[k] = k0 + k < ke ? ld_dev2(Pr + k0 + k) : make_float2(-INFINITY, 0.0f);
#pragma unroll
          for (int k = 0; k < 8; ++k) merge_sm(m, l, v[k].x, v[k].y);
        }
      }
      parts[q * BM + r] = make_float2(m, l);
      __syncthreads();
      if (t < BM && m0 + t < M) {
        float2 x = parts[t];
        for (int k = 1; k < NP; ++k) merge_sm(x.x, x.y, parts[k * BM + t].x, parts[k * BM + t].y);
        st_dev2(F + m0 + t, make_float2(x.x, 1.0f / x.y));
      }
      wait_stores();
      __syncthreads();
      if (t == 0) __hip_atomic_fetch_add(jw, (1ull << 32) - (uint64_t)T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // ------------------------------------------------ sweep 2: normalise, store
  i = 0;
  for (int tile = g; tile < tiles; tile += G, ++i) {
    const int rowblk = tile / T, tn = tile - rowblk * T;
    const int m0 = rowblk * BM, n0 = tn * BN;
    const bool more = tile + G < tiles;
    const int nt = more ? tile + G : 0;
    f32x16 acc[RB][CB];
    zero_acc(acc);
    main_loop<BM, BN, BK, false, RB, CB>(rg, rA, rB, s0, s1, m0, n0, more, (nt / T) * BM, (nt % T) * BN, acc, KT,
                                         wm, wn);
    if (t == 0) wait_generation(a.joins + rowblk, gens[i], a.err);
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = m0 + lrow + rb * 32;
      const float2 st = row < M ? ld_dev2(F + row) : make_float2(0.0f, 0.0f);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int col = n0 + lcol + cb * 32 + 8 * h;
          float o[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = __builtin_amdgcn_exp2f(acc[rb][cb][8 * h + e] * sc - st.x) * st.y;
          const u32x4 pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                            pack_bf16x2(o[6], o[7])};
          bst16(rY, (row < M && col < N) ? (uint32_t)(row * N + col) * 2u : kOOB, pk);
        }
      }
    }
  }
}

// Two bf16 lanes from two fp32 values, round to nearest even (one gfx950
// conversion instruction).
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// GEMM + row softmax by strips, for a reduction dimension of at most 128.
// A workgroup owns a strip: BM = 128 rows (32 per wave) by a contiguous run
// of BN = 128-column tiles.  Its Q rows stay in registers as MFMA operands;
// only the K tiles stream through a two-slot LDS ring.  Every wave owns whole
// rows of each tile, so per-tile row statistics are lane-local plus one lane
// exchange, and they accumulate online across the strip.
//   Sweep 1: strip statistics (max, sum of 2^(s - max)) per row, published
//   once; the last strip of a row block to arrive merges the block's strips
//   in order and publishes max + log2(sum) per row.
//   Sweep 2: after the row block's statistics are in (usually long before),
//   the strip is computed again, normalised (2^(s - max - log2 sum): the
//   division rides in the exponent) and stored as bf16.
// The strip is recomputed rather than held across the wait: with a short
// reduction dimension the second pass costs less than the exchange it hides.
constexpr int kSmBM = 128, kSmBN = 128, kSmBK = 128;

// One tile's contribution to this lane's running row statistics (m, l) in
// the base-2 domain, from the raw products acc (scaled by sc).  Chunk q =
// (cb, h) holds the 8 columns c0 + cb*32 + 8h + [0, 8), valid or not as a
// whole; RAGGED tiles mask the chunks past N, full tiles skip the tests.
// The extreme raw value (max for sc >= 0, min otherwise: scaling is monotone)
// comes from three-input NaN-propagating max / min trees over independent
// chunks, which take no canonicalising moves; a NaN product makes the row's
// sum NaN either way.
template <int CB, bool RAGGED>
__device__ __forceinline__ void sm_tile_stats(const f32x16 (&acc)[CB], int c0, int N, float sc, float& m, float& l) {
  bool ok[2 * CB];
#pragma unroll
  for (int q = 0; q < 2 * CB; ++q) ok[q] = !RAGGED || c0 + (q >> 1) * 32 + 8 * (q & 1) < N;
  auto mx = [](float x, float y) { return __builtin_elementwise_maximum(x, y); };
  auto mn = [](float x, float y) { return __builtin_elementwise_minimum(x, y); };
  float cm[2 * CB];
  const bool up = sc >= 0.0f;
#pragma unroll
  for (int q = 0; q < 2 * CB; ++q) {
    float e[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) e[k] = acc[q >> 1][8 * (q & 1) + k];
    const float x = up ? mx(mx(mx(e[0], e[1]), e[2]), mx(mx(mx(e[3], e[4]), e[5]), mx(e[6], e[7])))
                       : mn(mn(mn(e[0], e[1]), e[2]), mn(mn(mn(e[3], e[4]), e[5]), mn(e[6], e[7])));
    cm[q] = ok[q] ? x : (up ? -INFINITY : INFINITY);
  }
#pragma unroll
  for (int st = 1; st < 2 * CB; st *= 2)
#pragma unroll
    for (int q = 0; q + st < 2 * CB; q += 2 * st) cm[q] = up ? mx(cm[q], cm[q + st]) : mn(cm[q], cm[q + st]);
  const float ex = cm[0];
  if (ex == INFINITY || ex == -INFINITY) return;
  const float mnew = fmaxf(m, ex * sc);
  float cs[2 * CB];
#pragma unroll
  for (int q = 0; q < 2 * CB; ++q) {
    float e[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) e[k] = __builtin_amdgcn_exp2f(fmaf(acc[q >> 1][8 * (q & 1) + k], sc, -mnew));
    const float x = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    cs[q] = ok[q] ? x : 0.0f;
  }
#pragma unroll
  for (int st = 1; st < 2 * CB; st *= 2)
#pragma unroll
    for (int q = 0; q + st < 2 * CB; q += 2 * st) cs[q] += cs[q + st];
  l = l * __builtin_amdgcn_exp2f(m - mnew) + cs[0];
  m = mnew;
}

template <int KS, int MINB>
__global__ __launch_bounds__(kThreads, MINB) void k_gemm_sm3(GemmArgs a) {
  constexpr int BM = kSmBM, BN = kSmBN, BK = kSmBK;
  constexpr int CB = BN / 32;  // KS: 16-deep k-steps covering the reduction dimension
  constexpr int SLOT = BN * BK * 2;  // one K tile: BN keys x BK dims
  constexpr int LB = SLOT / 4096;    // 16-byte direct loads per lane per tile
  __shared__ __align__(16) char s0[SLOT];
  __shared__ __align__(16) char s1[SLOT];
  __shared__ uint32_t gens[kMaxRounds];
  __shared__ int last;

  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  const int M = (int)a.M, N = (int)a.N, D = (int)a.K;
  const int G = (int)gridDim.x;
  const int g = (int)xcd_local_id(blockIdx.x, (uint32_t)G);
  const int T = a.tiles_n;        // column tiles per row
  const int S = a.strips;         // strips per row block
  const int C = (T + S - 1) / S;  // tiles per strip
  const int units = a.tiles_m * S;
  if (g >= units) return;
  const __amdgpu_buffer_rsrc_t rA = rsrc(a.A, (uint32_t)(a.M * a.K * 2));
  const __amdgpu_buffer_rsrc_t rB = rsrc(a.B, (uint32_t)(a.N * a.K * 2));
  const __amdgpu_buffer_rsrc_t rY = rsrc(a.Y, (uint32_t)(a.M * a.N * 2));
  const float sc = a.scale * kLog2e;
  float2* P = reinterpret_cast<float2*>(a.partials);
  float2* F = reinterpret_cast<float2*>(a.finals);

  // direct loads of K tile j (keys j*BN .., all dims) into a slot.  The
  // lane's byte offset within a tile is fixed (kOOB past the reduction
  // dimension); keys past N fall outside the buffer's range and read zero.
  // Load q puts key 16q + kl (kl = 4w + lane/16) at chunk lane % 16; the
  // sigma swizzle of that row depends on q only through q & 1, so two
  // per-lane offsets serve every load (plus 16q keys, uniform).
  static_assert(BK == 128, "16 keys per 4 KB load, 16 chunks per row");
  uint32_t koff[2];
  {
    const int kl = 4 * w + (lane >> 4), pc = lane & 15;
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int gk = 8 * swz_sigma<BK>(kl + 16 * par, pc);
      koff[par] = gk < D ? (uint32_t)(kl * D + gk) * 2u : kOOB;
    }
  }
  auto load_tile = [&](char* slot, int j) {
    const uint32_t base = (uint32_t)(j * BN) * (uint32_t)D * 2u;
#pragma unroll
    for (int q = 0; q < LB; ++q) g2l16(rB, slot + (q * 4 + w) * 1024, koff[q & 1] + base + (uint32_t)(32 * q * D));
  };
  // strip u's first tile, and the tile that follows tile j of strip u
  auto strip_first = [&](int u) { return (u % S) * C; };
  auto strip_end = [&](int u) { return min(T, (u % S) * C + C); };

  // one tile's MFMAs from a slot: acc[cb] += K-tile rows (permuted) x Q rows;
  // step ks+1's fragments are all read before step ks's MFMAs issue (hard
  // scheduling barriers keep the two register sets apart)
  auto mma_tile = [&](const char* slot, const bf16x8_t (&qf)[KS], f32x16 (&acc)[CB]) {
    bf16x8_t kf[2][CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int key = cb * 32 + sigma(l32);
      kf[0][cb] = *reinterpret_cast<const bf16x8_t*>(slot + key * (BK * 2) + 16 * swz_sigma<BK>(key, hl));
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < KS) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int key = cb * 32 + sigma(l32);
          kf[cur ^ 1][cb] =
              *reinterpret_cast<const bf16x8_t*>(slot + key * (BK * 2) + 16 * swz_sigma<BK>(key, 2 * (ks + 1) + hl));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[cur][cb], qf[ks], acc[cb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto load_q = [&](int m0, bf16x8_t (&qf)[KS]) {
    const int row = m0 + w * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int k = 16 * ks + 8 * hl;
      qf[ks] = __builtin_bit_cast(bf16x8_t, bld16(rA, (row < M && k < D) ? (uint32_t)(row * D + k) * 2u : kOOB));
    }
  };

  // the tile stream: sweep 1 over this workgroup's strips, then sweep 2 over
  // the same strips; stage st of the stream lives in slot st & 1
  int st = 0;
  load_tile(s0, strip_first(g));
  auto next_tile = [&](int sweep, int u, int j, int* nj) -> bool {
    if (j + 1 < strip_end(u)) { *nj = j + 1; return true; }
    if (u + G < units) { *nj = strip_first(u + G); return true; }
    if (sweep == 1) { *nj = strip_first(g); return true; }
    return false;
  };
  // wait for stage st, free the other slot, prefetch the next stage into it,
  // then run the tile from stage st's slot.  `stored`: the previous step
  // issued the 8 output stores of its tile after this stage's prefetch; the
  // vector-memory counter retires in issue order, so waiting down to those 8
  // completes the prefetch while the stores keep draining under this tile's
  // MainLoop (they must be done only by the wait one step later).
  constexpr int kStoresPerTile = 2 * CB;
  auto step = [&](int sweep, int u, int j, const bf16x8_t (&qf)[KS], f32x16 (&acc)[CB], bool stored) {
    if (stored) wait_vm<kStoresPerTile>();
    else wait_vm<0>();
    __syncthreads();
    int nj = 0;
    const bool more = next_tile(sweep, u, j, &nj);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[cb][r] = 0.0f;
    if (st & 1) {
      if (more) load_tile(s0, nj);
      mma_tile(s1, qf, acc);
    } else {
      if (more) load_tile(s1, nj);
      mma_tile(s0, qf, acc);
    }
    ++st;
  };

  // ------------------------------------------------ sweep 1: statistics
  int i = 0;
  for (int u = g; u < units; u += G, ++i) {
    const int rowblk = u / S, m0 = rowblk * BM;
    bf16x8_t qf[KS];
    load_q(m0, qf);
    float m = -INFINITY, l = 0.0f;  // running, base-2 domain, this lane's row
    for (int j = strip_first(u); j < strip_end(u); ++j) {
      f32x16 acc[CB];
      step(1, u, j, qf, acc, false);
      // chunk (cb, h) of this lane's row holds columns j*BN + cb*32 + 16*hl + 8*h + [0, 8)
      const int c0 = j * BN + 16 * hl;
      if (j * BN + BN <= N) sm_tile_stats<CB, false>(acc, c0, N, sc, m, l);
      else sm_tile_stats<CB, true>(acc, c0, N, sc, m, l);
    }
    merge_sm(m, l, __shfl_xor(m, 32, kWave), __shfl_xor(l, 32, kWave));
    const int row = m0 + w * 32 + l32;
    if (hl == 0 && row < M) st_dev2(P + (size_t)row * S + (u % S), make_float2(m, l));
    wait_stores();
    __syncthreads();
    uint64_t* jw = a.joins + rowblk;
    if (t == 0) {
      const uint64_t old = __hip_atomic_fetch_add(jw, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = ((uint32_t)old == (uint32_t)(S - 1)) ? 1 : 0;
      gens[i] = (uint32_t)(old >> 32);
    }
    __syncthreads();
    if (last) {
      // merge the block's strips per row, in strip order, all loads in flight
      if (t < BM && m0 + t < M) {
        const float2* Pr = P + (size_t)(m0 + t) * S;
        float mm = -INFINITY, ll = 0.0f;
        for (int k0 = 0; k0 < S; k0 += 8) {
          float2 v[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) v[k] = k0 + k < S ? ld_dev2(Pr + k0 + k) : make_float2(-INFINITY, 0.0f);
#pragma unroll
          for (int k = 0; k < 8; ++k) merge_sm(mm, ll, v[k].x, v[k].y);
        }
        // the row's offset max + log2(sum): sweep 2 normalises inside the exponent
        st_dev2(F + m0 + t, make_float2(mm + __builtin_amdgcn_logf(ll), 0.0f));
      }
      wait_stores();
      __syncthreads();
      if (t == 0) __hip_atomic_fetch_add(jw, (1ull << 32) - (uint64_t)S, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // ------------------------------------------------ sweep 2: normalise, store
  i = 0;
  for (int u = g; u < units; u += G, ++i) {
    const int rowblk = u / S, m0 = rowblk * BM;
    bf16x8_t qf[KS];
    load_q(m0, qf);
    if (t == 0) wait_generation(a.joins + rowblk, gens[i], a.err);
    __syncthreads();
    const int row = m0 + w * 32 + l32;
    const float off = row < M ? ld_dev2(F + row).x : 0.0f;
    for (int j = strip_first(u); j < strip_end(u); ++j) {
      f32x16 acc[CB];
      step(2, u, j, qf, acc, j > strip_first(u));
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int col = j * BN + cb * 32 + 16 * hl + 8 * h;
          float o[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = __builtin_amdgcn_exp2f(fmaf(acc[cb][8 * h + e], sc, -off));
          const u32x4 pk = {cvt_bf16x2(o[0], o[1]), cvt_bf16x2(o[2], o[3]), cvt_bf16x2(o[4], o[5]),
                            cvt_bf16x2(o[6], o[7])};
          bst16(rY, (row < M && col < N) ? (uint32_t)(row * N + col) * 2u : kOOB, pk);
        }
    }
  }
}


// Back-to-back GEMM with the row softmax between, O = softmax(scale Q.K^T).V
// ([ComFuse] "B2BGEMM": S_tile = F(P_tile), eq. 3; partial products
// S_tile.W2_tile over the contraction dimension, eq. 4; their sum at the
// commit, eq. 5; the W1 and W2 tiles share one circular buffer).  F is the
// cross-tile row softmax.  A workgroup owns a strip (a row block's run of
// 64-key tiles) and merges F's row statistics online, tile by tile, as the
// pages' statistics exchange does between workgroups: per tile, K block j
// (first MatMul, P = Q.K_j^T), then V block j, where the row max rises to
// include the tile (the output accumulator and the row sum are scaled by
// 2^(old max - new max)), the tile 2^(P*sc - max) goes from the accumulator
// straight into bf16 operand fragments and meets V_j in the second MatMul,
// and its row sums accumulate beside.  A lane holds 16 consecutive keys of
// its row, so the second MatMul's k-order is permuted to match (k-slots 0-7
// take keys 0-7 of lanes 0-31 and keys 16-23 of lanes 32-63, and so on) and
// V's transposed fragment reads follow it.
// Commit: each strip publishes its partial output with its (max, sum) per
// row (the tile goes through LDS so every store writes whole 1 KB runs);
// after the row block's join every strip sums its share of the rows over the
// strips, in strip order, each weighted by 2^(strip max - block max), divides
// by the equally weighted sums and stores O.  Exact in real arithmetic.
// One workgroup of 8 waves per CU (32 rows per wave, 256-row strips): the
// strip's Q rows sit in LDS, and the K / V blocks stream through a 4-slot
// ring that holds two tiles (one computed, the next in flight; one barrier
// per tile), each slot its own LDS object so the compiler can tell the slot
// being read from the ones being filled.
template <int KS, int NS>
__global__ __launch_bounds__(kB2bThreads, 1) void k_gemm_b2b(GemmArgs a) {
  constexpr int BM = kB2bBM, BN = kB2bBN, BK = kB2bBK, NW = kB2bWaves, THREADS = kB2bThreads;
  constexpr int CB = BN / 32;            // 32-key blocks per tile
  constexpr int DV = 128, NB = DV / 32;  // output columns held (zero past Dv)
  constexpr int SLOT = BN * BK * 2;      // one K block (BN keys x BK dims) or V block (BN keys x DV)
  constexpr int LPS = SLOT / (NW * 1024);  // 16-byte direct loads per lane per block
  static_assert(SLOT == BN * DV * 2 && LPS * NW * 1024 == SLOT && BK == 128, "block shapes");
  static_assert(NS == 4, "two tiles of K and V blocks");
  __shared__ __align__(16) char sq[BM * BK * 2];  // the strip's Q rows
  __shared__ __align__(16) char r0[SLOT];
  __shared__ __align__(16) char r1[SLOT];
  __shared__ __align__(16) char r2[SLOT];
  __shared__ __align__(16) char r3[SLOT];
  __shared__ uint32_t gen2;
  // slot i of the ring (i is a constant wherever a block is computed on)
  auto ring = [&](int i) -> char* { return i == 0 ? r0 : i == 1 ? r1 : i == 2 ? r2 : r3; };

  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  const int M = (int)a.M, N = (int)a.N, D = (int)a.K, Dv = (int)a.Dv;
  const int G = (int)gridDim.x;
  const int g = (int)xcd_local_id(blockIdx.x, (uint32_t)G);
  const int T = a.tiles_n;        // 64-key tiles per row
  const int S = a.strips;         // strips per row block
  const int C = (T + S - 1) / S;  // tiles per strip
  const int units = a.tiles_m * S;
  if (g >= units) return;
  const __amdgpu_buffer_rsrc_t rA = rsrc(a.A, (uint32_t)(a.M * a.K * 2));
  const __amdgpu_buffer_rsrc_t rB = rsrc(a.B, (uint32_t)(a.N * a.K * 2));
  const __amdgpu_buffer_rsrc_t rV = rsrc(a.V, (uint32_t)(a.N * a.Dv * 2));
  const __amdgpu_buffer_rsrc_t rO = rsrc(a.Y, (uint32_t)(a.M * a.Dv * 2));
  // partial outputs, strip-major: [S][M][DV] bf16, then (max, sum) [S][M] float2
  const __amdgpu_buffer_rsrc_t rOp = rsrc(a.opart, (uint32_t)(a.M * S * DV * 2));
  float2* const Lp = reinterpret_cast<float2*>(reinterpret_cast<char*>(a.opart) + (size_t)a.M * S * DV * 2);
  const float sc = a.scale * kLog2e;

  // Direct loads: load q of a block puts key 32q + kl (kl = 4w + lane/16 <
  // 32) at 16-byte chunk lane % 16 of that key's 256-byte row; the row's
  // swizzle (sigma rows for K, 64-byte segments for V) does not depend on q,
  // so one per-lane offset serves every load.  Columns past D (K) or Dv (V)
  // and keys past N read zero.
  uint32_t koff, voff;
  {
    const int kl = 4 * w + (lane >> 4), pc = lane & 15;
    const int gk = 8 * swz_sigma<BK>(kl, pc);
    koff = gk < D ? (uint32_t)(kl * D + gk) * 2u : kOOB;
    const int col = ((pc * 16) ^ nn_mask(kl)) / 2;
    voff = col < Dv ? (uint32_t)(kl * Dv + col) * 2u : kOOB;
  }
  auto load_k = [&](char* slot, int j) {
    const uint32_t base = (uint32_t)(j * BN) * (uint32_t)D * 2u;
#pragma unroll
    for (int q = 0; q < LPS; ++q) g2l16(rB, slot + (q * NW + w) * 1024, koff + base + (uint32_t)(64 * q * D));
  };
  auto load_v = [&](char* slot, int j) {
    const uint32_t base = (uint32_t)(j * BN) * (uint32_t)Dv * 2u;
#pragma unroll
    for (int q = 0; q < LPS; ++q) g2l16(rV, slot + (q * NW + w) * 1024, voff + base + (uint32_t)(64 * q * Dv));
  };
  // The strip's Q rows: row r's 16-byte chunk c at r*256 + 16*(c ^ r%16), so
  // 16 lanes reading 16 rows at one chunk hit 16 distinct bank slots.  Load q
  // fills rows 32q + 4w + lane/16; the chunk and its swizzle do not depend on
  // q, so one per-lane offset serves every load (no per-load address state to
  // keep live).  Rows past M lie beyond the descriptor's range and read zero.
  uint32_t qoff;
  bool qok;
  {
    const int r = 4 * w + (lane >> 4), c = (lane & 15) ^ (r & 15);
    qok = 8 * c < D;
    qoff = (uint32_t)(r * D + 8 * c) * 2u;
  }
  auto load_q = [&](int m0) {
    uint32_t o = qoff + (uint32_t)m0 * (uint32_t)D * 2u;
    // opaque, so the per-load sums are formed here and not hoisted out of
    // the strip loop as eight live registers (which would spill)
    asm volatile("" : "+v"(o));
#pragma unroll
    for (int q = 0; q < BM * BK * 2 / (NW * 1024); ++q)
      g2l16(rA, sq + (q * NW + w) * 1024, qok ? o + (uint32_t)(64 * q * D) : kOOB);
  };
  // First MatMul of one tile: acc[cb] += K rows (sigma-permuted) x Q rows;
  // step ks+1's K and Q fragments are read before step ks's MFMAs issue
  const int qr = w * 32 + l32;
  auto mma_qk = [&](const char* slot, f32x16 (&acc)[CB]) {
    const char* qrow = sq + qr * 256;
    bf16x8_t kf[2][CB], qv[2];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int key = cb * 32 + sigma(l32);
      kf[0][cb] = *reinterpret_cast<const bf16x8_t*>(slot + key * (BK * 2) + 16 * swz_sigma<BK>(key, hl));
    }
    qv[0] = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * (hl ^ (qr & 15)));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < KS) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int key = cb * 32 + sigma(l32);
          kf[cur ^ 1][cb] =
              *reinterpret_cast<const bf16x8_t*>(slot + key * (BK * 2) + 16 * swz_sigma<BK>(key, 2 * (ks + 1) + hl));
        }
        qv[cur ^ 1] = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * ((2 * (ks + 1) + hl) ^ (qr & 15)));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[cur][cb], qv[cur], acc[cb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // V fragment for key block cb, half q, column block nb: 8 consecutive
  // (permuted) keys of one column by two transposed reads.  The lane reads
  // key k = cb*32 + 16*(lane/32) + 8q + 4hh + e, column n = nb*32 + c (e, c
  // from the lane): k % 4 = e, so the segment XOR is (nb ^ e) * 64 and the
  // byte offset is a per-lane base per nb plus a constant.
  uint32_t vb[NB];
  {
    const int Gq = lane >> 4, L = lane & 15, e = L >> 2, cc = L & 3;
    const int clow = 2 * (16 * (cc & 1) + 8 * (Gq & 1) + 4 * (cc >> 1));  // < 64
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) vb[nb] = (uint32_t)((16 * (Gq >> 1) + e) * (DV * 2) + ((nb ^ e) << 6) + clow);
  }
  auto vfrag = [&](const char* slot, int cb, int q, int nb) -> bf16x8_t {
    bf16x4_t h[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4_t*)(slot + vb[nb] + (cb * 32 + 8 * q + 4 * hh) * (DV * 2)));
    return __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // Tile j of the strip: the row's reference max m moves only when the tile
  // exceeds it by more than 2^8 (both lanes of a row agree: one exchange);
  // then oacc and l are scaled by 2^(m_old - m_new).  Exponents stay at most
  // 2^8 (bf16 and fp32 hold them), and the result is the same in real
  // arithmetic whichever reference is used.  Then E = 2^(P*sc - m) (zero on
  // keys past N) into bf16 fragments, one 32-key block at a time, each
  // followed by its MFMAs; the lane's share of the row sum accumulates in fp32
  auto mma_ev = [&](const char* slot, const f32x16 (&acc)[CB], float& m, int j, f32x16 (&oacc)[NB], float& l) {
    float tx = sc >= 0.0f ? -INFINITY : INFINITY;  // max (or min) of the raw scores
    const bool whole = (j + 1) * BN <= N;           // every key of the tile is valid (uniform)
    if (sc >= 0.0f && whole) {
      // a tree of three-input NaN-propagating maxima over 8-value chunks: no
      // long dependency chain and no canonicalising moves (a NaN score makes
      // the row NaN either way)
      auto mx = [](float x, float y) { return __builtin_elementwise_maximum(x, y); };
      float cm[2 * CB];
#pragma unroll
      for (int q = 0; q < 2 * CB; ++q) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = acc[q >> 1][8 * (q & 1) + e];
        cm[q] = mx(mx(mx(v[0], v[1]), v[2]), mx(mx(mx(v[3], v[4]), v[5]), mx(v[6], v[7])));
      }
#pragma unroll
      for (int d = 1; d < 2 * CB; d *= 2)
#pragma unroll
        for (int q = 0; q + d < 2 * CB; q += 2 * d) cm[q] = mx(cm[q], cm[q + d]);
      tx = cm[0];
    } else if (sc >= 0.0f) {
#pragma unroll
      for (int q = 0; q < 2 * CB; ++q)
        if (j * BN + (q >> 1) * 32 + 16 * hl + 8 * (q & 1) < N)
#pragma unroll
          for (int e = 0; e < 8; ++e) tx = fmaxf(tx, acc[q >> 1][8 * (q & 1) + e]);
    } else {
#pragma unroll
      for (int q = 0; q < 2 * CB; ++q)
        if (j * BN + (q >> 1) * 32 + 16 * hl + 8 * (q & 1) < N)
#pragma unroll
          for (int e = 0; e < 8; ++e) tx = fminf(tx, acc[q >> 1][8 * (q & 1) + e]);
    }
    float tm = (tx == INFINITY || tx == -INFINITY) ? -INFINITY : tx * sc;  // base-2 domain
    tm = fmaxf(tm, __shfl_xor(tm, 32, kWave));
    if (tm > m + 8.0f) {  // raise the reference (the first valid tile always does)
      const float corr = __builtin_amdgcn_exp2f(m - tm);  // 0 while m = -inf
      l *= corr;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[nb][r] *= corr;
      m = tm;
    }
    // (m = -inf only before the row's first key: then E is zero; the MFMAs
    // below always run for the whole wave)
    const bool live = m != -INFINITY;
    const float mn = live ? m : 0.0f;
    // a whole tile of valid keys needs no per-chunk masking
    const bool full = live && whole;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      bf16x8_t sf[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float y[8];
        if (full) {
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = __builtin_amdgcn_exp2f(fmaf(acc[cb][8 * q + e], sc, -mn));
        } else {
          const bool ok = live && j * BN + cb * 32 + 16 * hl + 8 * q < N;
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = ok ? __builtin_amdgcn_exp2f(fmaf(acc[cb][8 * q + e], sc, -mn)) : 0.0f;
        }
        l += ((y[0] + y[1]) + (y[2] + y[3])) + ((y[4] + y[5]) + (y[6] + y[7]));
        const u32x4 pk = {cvt_bf16x2(y[0], y[1]), cvt_bf16x2(y[2], y[3]), cvt_bf16x2(y[4], y[5]),
                          cvt_bf16x2(y[6], y[7])};
        sf[q] = __builtin_bit_cast(bf16x8_t, pk);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        bf16x8_t vf[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) vf[nb] = vfrag(slot, cb, q, nb);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[nb], sf[q], oacc[nb], 0, 0, 0);
      }
    }
  };
  auto strip_first = [&](int u) { return (u % S) * C; };
  auto strip_len = [&](int u) { return min(T, (u % S) * C + C) - (u % S) * C; };

  // ------------------------------------------------ the strips
  int qloaded = -1;  // row block whose Q rows are in LDS
  for (int u = g; u < units; u += G) {
    const int rowblk = u / S, m0 = rowblk * BM, su = u % S, j0 = strip_first(u);
    __syncthreads();  // every wave is done with the LDS of the previous strip
    if (qloaded != rowblk) load_q(m0);
    qloaded = rowblk;
    const int row = m0 + qr;
    float m = -INFINITY;  // running row max, base-2 domain
    f32x16 oacc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[nb][r] = 0.0f;
    float lsum = 0.0f;
    f32x16 acc[CB];
    // tile x of the strip: K block in slot 2(x % 2), V block in slot 2(x % 2) + 1.
    // One barrier per tile publishes both blocks of tile x and retires tile
    // x - 1's slots, into which tile x + 1 is issued at once (one tile ahead);
    // the Q rows, issued before tile 0, are covered by its wait
    const int len = strip_len(u);  // >= 1: the planner gives every strip a tile
    if (len > 0) {
      load_k(ring(0), j0);
      load_v(ring(1), j0);
    }
    for (int x0 = 0; x0 < len; x0 += 2) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int x = x0 + h;
        if (x >= len) break;
        wait_vm<0>();
        __syncthreads();
        if (x + 1 < len) {
          load_k(ring(2 * (h ^ 1)), j0 + x + 1);
          load_v(ring(2 * (h ^ 1) + 1), j0 + x + 1);
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[cb][r] = 0.0f;
        mma_qk(ring(2 * h), acc);
        mma_ev(ring(2 * h + 1), acc, m, j0 + x, oacc, lsum);
      }
    }
    lsum += __shfl_xor(lsum, 32, kWave);  // the row's sum over the strip (relative to m)
    // this lane's output row, columns nb*32 + 16*hl + [0, 16)
    if (S == 1) {
      const float inv = 1.0f / lsum;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int col = nb * 32 + 16 * hl + 8 * h;
          float o[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = oacc[nb][8 * h + e] * inv;
          const u32x4 pk = {cvt_bf16x2(o[0], o[1]), cvt_bf16x2(o[2], o[3]), cvt_bf16x2(o[4], o[5]),
                            cvt_bf16x2(o[6], o[7])};
          bst16(rO, (row < M && col < Dv) ? (uint32_t)(row * Dv + col) * 2u : kOOB, pk);
        }
      continue;
    }
    // publish the strip's partial output, rounded to bf16, through LDS (now
    // idle): wave w's 32 rows go to a region of its own (Q rows for waves
    // 0-3, ring slots for waves 4-7), 16-byte chunk k (8 columns) of row r
    // at r*256 + 16*(k ^ (r % 16)), then back out as whole rows, 1 KB per
    // store instruction
    __syncthreads();  // every wave is done with the ring and the Q rows
    // (the region is picked at run time from separate LDS objects, so the
    // pointer is cast back to the LDS address space: the stores and loads
    // below are then LDS instructions with 32-bit addresses, not flat ones)
    lds_char_t* const stage = (lds_char_t*)(w < 4 ? sq + w * 16384 : ring(w - 4));
    static_assert(NS >= 4 && SLOT == 16384 && BM * BK * 2 == 4 * 16384, "one staging region per wave");
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k8 = nb * 4 + 2 * hl + h;  // 16-byte chunk index of columns 8*k8 .. +7
        const u32x4 v = {cvt_bf16x2(oacc[nb][8 * h], oacc[nb][8 * h + 1]), cvt_bf16x2(oacc[nb][8 * h + 2], oacc[nb][8 * h + 3]),
                         cvt_bf16x2(oacc[nb][8 * h + 4], oacc[nb][8 * h + 5]), cvt_bf16x2(oacc[nb][8 * h + 6], oacc[nb][8 * h + 7])};
        *reinterpret_cast<lds_u32x4_t*>(stage + l32 * 256 + 16 * (k8 ^ (l32 & 15))) = v;
      }
    if (hl == 0 && row < M) st_dev2(Lp + (size_t)su * M + row, make_float2(m, lsum));
    __syncthreads();
#pragma unroll 4
    for (int it = 0; it < 8; ++it) {
      const int idx = it * 64 + lane, r = idx >> 4, k8 = idx & 15;
      const int orow = m0 + w * 32 + r;
      const u32x4 v = *reinterpret_cast<const lds_u32x4_t*>(stage + r * 256 + 16 * (k8 ^ (r & 15)));
      bst16_dev(rOp, orow < M ? (uint32_t)((((size_t)su * M + orow) * DV + 8 * k8) * 2) : kOOB, v);
    }
    wait_stores();
    __syncthreads();
    uint64_t* jw2 = a.joins + a.tiles_m + rowblk;
    if (t == 0) {
      const uint64_t old = __hip_atomic_fetch_add(jw2, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((uint32_t)old == (uint32_t)(S - 1))
        __hip_atomic_fetch_add(jw2, (1ull << 32) - (uint64_t)S, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      gen2 = (uint32_t)(old >> 32);
    }
    __syncthreads();
    if (t == 0) wait_generation(jw2, gen2, a.err);
    __syncthreads();
    // strip su sums rows [su*R, su*R + R) of the block over the strips, in
    // strip order, merging (max, sum, output) online: each strip weighted by
    // 2^(its max - the running max), the running terms rescaled when the max
    // rises; 8 columns per item, every load of 8 strips in flight at once
    const int R = (BM + S - 1) / S;
    for (int it = t; it < R * (DV / 8); it += THREADS) {
      const int r = su * R + it / (DV / 8), c8 = (it % (DV / 8)) * 8;
      const int orow = m0 + r;
      if (r >= BM || orow >= M || c8 >= Dv) continue;
      float o[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
      float mb = -INFINITY, ls = 0.0f;
      for (int sk = 0; sk < S; sk += 8) {
        u32x4 v[8];
        float2 lv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          v[k] = bld16_dev(rOp, sk + k < S ? (uint32_t)((((size_t)(sk + k) * M + orow) * DV + c8) * 2) : kOOB);
          lv[k] = sk + k < S ? ld_dev2(Lp + (size_t)(sk + k) * M + orow) : make_float2(-INFINITY, 0.0f);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (lv[k].x == -INFINITY) continue;  // a strip with no key (or past S)
          if (lv[k].x > mb) {
            const float sdn = __builtin_amdgcn_exp2f(mb - lv[k].x);  // 0 while mb = -inf
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] *= sdn;
            ls *= sdn;
            mb = lv[k].x;
          }
          const float wgt = __builtin_amdgcn_exp2f(lv[k].x - mb);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t x = v[k][e >> 1];  // bf16 pair: column e & ~1 low, e | 1 high
            o[e] = fmaf(wgt, __uint_as_float((e & 1) ? (x & 0xFFFF0000u) : (x << 16)), o[e]);
          }
          ls = fmaf(wgt, lv[k].y, ls);
        }
      }
      const float inv = 1.0f / ls;
      const u32x4 pk = {cvt_bf16x2(o[0] * inv, o[1] * inv), cvt_bf16x2(o[2] * inv, o[3] * inv),
                        cvt_bf16x2(o[4] * inv, o[5] * inv), cvt_bf16x2(o[6] * inv, o[7] * inv)};
      bst16(rO, (uint32_t)(orow * Dv + c8) * 2u, pk);
    }
  }
}

// Tile of logical workgroup g in round r.  Round r holds the tiles
// [r*G, (r+1)*G) of the row-major tile order, whatever the mapping, so each
// round's tile set (and with it every argument about which rounds a row
// block spans) is that of the linear order.  Within a full round of whole row
// blocks, XCD x (logical ids [x*G/8, (x+1)*G/8), see xcd_local_id) takes a
// compact block of (rows/sa) row blocks by (T/sb) column tiles, so its L2
// holds that block's A rows and W columns instead of every W column; an XCD
// keeps the same column slice from round to round.  Other rounds: linear.
__device__ __forceinline__ int round_tile(int g, int r, int G, int T, int tiles, int sa, int sb) {
  const int base = r * G;
  if (base + g >= tiles) return -1;
  if (sa == 0 || base + G > tiles) return base + g;
  const int per = G >> 3;
  const int x = g / per, k = g - x * per;
  const int brow = G / T / sa, bcol = T / sb;  // brow * bcol == per
  return base + ((x / sb) * brow + k / bcol) * T + (x % sb) * bcol + k % bcol;
}

// GEMM + bias + residual + LayerNorm with each tile's join waited on only
// after the NEXT tile's MainLoop (PIPE): a workgroup computes tile j,
// publishes its row statistics and arrives (the last member of the row block
// merges them), computes tile j+1, and only then waits for tile j's block,
// normalises and stores it.  Deadlock-free while every workgroup is resident
// and a row block's tiles span at most two rounds: a workgroup never waits
// before it has published the tile after the one it waits for.  Without PIPE
// (tiles too large for two accumulator sets) each tile is finished before
// the next begins, and whole row blocks fall in one round.
template <int BM, int BN, int BK, int WGM, int MINB, int NWAVES, bool PIPE, int NS>
__global__ __launch_bounds__(NWAVES * 64, MINB) void k_gemm_ln2(GemmArgs a) {
  using RG = Ring<BM, BN, BK, true, NWAVES>;
  constexpr int THREADS = NWAVES * 64;
  constexpr int WGN = NWAVES / WGM;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int RB = WM / 32, CB = WN / 32;
  constexpr int NP = THREADS / BM;
  static_assert(BM <= THREADS && THREADS % BM == 0 && WM % 32 == 0 && WN % 32 == 0, "tile");
  // ring slots: separate objects (unused ones shrink to a placeholder)
  __shared__ __align__(16) char s0[RG::STAGE_BYTES];
  __shared__ __align__(16) char s1[RG::STAGE_BYTES];
  __shared__ __align__(16) char s2[NS > 2 ? RG::STAGE_BYTES : 16];
  __shared__ __align__(16) char s3[NS > 3 ? RG::STAGE_BYTES : 16];
  static_assert(NS >= 2 && NS <= 4, "ring depth");
  // epilogue scratch: red (WGN x BM), parts (THREADS), stat (BM), vec (this
  // tile's bias | gamma | beta slices, zero past N).  One tile at a time, the
  // ring is idle during the epilogue, so the scratch lives in slot 0 when it
  // fits (more workgroups per CU); pipelined, it has its own LDS.
  constexpr int SCR = (WGN * BM + THREADS) * 16 + BM * 8 + 3 * BN * 4;
  constexpr bool ALIAS = !PIPE && SCR <= RG::STAGE_BYTES;
  __shared__ __align__(16) char scr_own[ALIAS ? 16 : SCR];
  char* const scr = ALIAS ? s0 : scr_own;
  float4* const red = reinterpret_cast<float4*>(scr);
  float4* const parts = red + WGN * BM;
  float2* const stat = reinterpret_cast<float2*>(parts + THREADS);
  float* const vec = reinterpret_cast<float*>(stat + BM);
  __shared__ uint32_t gen_sh;

  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int wm = w / WGN, wn = w % WGN;
  const int hl = lane >> 5, l32 = lane & 31;
  const int lrow = wm * WM + l32, lcol = wn * WN + 16 * hl;
  const int M = (int)a.M, N = (int)a.N;
  const int KT = (int)((a.K + BK - 1) / BK);
  const int G = (int)gridDim.x;
  const int g = (int)xcd_local_id(blockIdx.x, (uint32_t)G);
  const int T = a.tiles_n;
  const int tiles = a.tiles_m * T;
  if (g >= tiles) return;
  const __amdgpu_buffer_rsrc_t rA = rsrc(a.A, (uint32_t)(a.M * a.K * 2));
  const __amdgpu_buffer_rsrc_t rB = rsrc(a.B, (uint32_t)(a.N * a.K * 2));
  const __amdgpu_buffer_rsrc_t rY = rsrc(a.Y, (uint32_t)(a.M * a.N * 2));
  const __amdgpu_buffer_rsrc_t rR = rsrc(a.R, a.R ? (uint32_t)(a.M * a.N * 2) : 0u);  // no residual: reads zero
  const __amdgpu_buffer_rsrc_t rBias = rsrc(a.bias, (uint32_t)(a.N * 4));
  const __amdgpu_buffer_rsrc_t rGam = rsrc(a.gamma, (uint32_t)(a.N * 4));
  const __amdgpu_buffer_rsrc_t rBet = rsrc(a.beta, (uint32_t)(a.N * 4));
  // partials: (mean, M2) per row and column tile, 8 bytes; a tile's count
  // is its number of valid columns
  const int T2 = (T + 1) & ~1;  // row stride in partials, even: 16-byte aligned pairs
  const __amdgpu_buffer_rsrc_t rP = rsrc(a.partials, (uint32_t)(a.M * T2 * 8));
  const RG rg(a);
  char* const all_slots[4] = {s0, s1, s2, s3};
  char* sl[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) sl[q] = all_slots[q];
  bool staged = false;  // the next tile's first stages are already in the ring

  // MainLoop, u = acc + bias + R, tile statistics, publish and arrive.
  // Returns the generation the tile's row block arrived in.
  auto produce = [&](f32x16(&acc)[RB][CB], int tile, int next_tile) -> uint32_t {
    const int rowblk = tile / T, tn = tile - rowblk * T;
    const int m0 = rowblk * BM, n0 = tn * BN;
    const bool more = next_tile >= 0;
    const int nt = more ? next_tile : 0;
    zero_acc(acc);
    if (!staged) {
      __syncthreads();  // every wave is done with the ring
      prologue_ns<BM, BN, BK, true, NWAVES, NS>(rg, rA, rB, sl, m0, n0, KT);
    }
    const bool pre = PIPE && more && KT % NS == 0;
    main_loop_ns<BM, BN, BK, true, RB, CB, NWAVES, NS>(rg, rA, rB, sl, m0, n0, pre, (nt / T) * BM, (nt % T) * BN,
                                                       acc, KT, wm, wn);
    staged = pre;
    if constexpr (ALIAS) __syncthreads();  // every wave is done with slot 0 before the scratch in it is written
    // stage 1: u = acc + bias_j + R_ij in the accumulator registers (zero on
    // columns past N), then the lane's (count, mean, M2) over valid columns
    float n_[RB], mu[RB], m2[RB];
    {
      // every residual load of the tile in one round trip, and the tile's bias
      // slice into LDS
      constexpr int CBB = CB;
      for (int c = t; c < BN; c += THREADS) vec[c] = bld4f(rBias, n0 + c < N ? (uint32_t)(n0 + c) * 4u : kOOB);
      __syncthreads();
#pragma unroll
      for (int cb0 = 0; cb0 < CB; cb0 += CBB) {
        u32x4 rr[RB][CBB][2];
#pragma unroll
        for (int cq = 0; cq < CBB; ++cq)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int col = n0 + lcol + (cb0 + cq) * 32 + 8 * h;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
              const int row = m0 + lrow + rb * 32;
              rr[rb][cq][h] = bld16(rR, (col < N && row < M) ? (uint32_t)(row * N + col) * 2u : kOOB);
            }
          }
#pragma unroll
        for (int cq = 0; cq < CBB; ++cq) {
          const int cb = cb0 + cq;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int cl = lcol + cb * 32 + 8 * h;
            const bool ok = n0 + cl < N;
            const float4 b0 = *reinterpret_cast<const float4*>(vec + cl);
            const float4 b1 = *reinterpret_cast<const float4*>(vec + cl + 4);
            const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const uint32_t wv = rr[rb][cq][h][e >> 1];
                const float u = acc[rb][cb][8 * h + e] + bv[e] + ((e & 1) ? bf16_hi(wv) : bf16_lo(wv));
                acc[rb][cb][8 * h + e] = ok ? u : 0.0f;
              }
            }
          }
        }
      }
    }
    int nvalid = 0;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int h = 0; h < 2; ++h) nvalid += (n0 + lcol + cb * 32 + 8 * h < N) ? 8 : 0;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float sum = 0.0f;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += acc[rb][cb][r];
      const float mean = nvalid > 0 ? sum / (float)nvalid : 0.0f;
      float q2 = 0.0f;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float d = (n0 + lcol + cb * 32 + (r & 8) < N) ? acc[rb][cb][r] - mean : 0.0f;
          q2 = fmaf(d, d, q2);
        }
      n_[rb] = (float)nvalid;
      mu[rb] = mean;
      m2[rb] = q2;
    }
    tile_merge_ln<BM, WGN, RB>(n_, mu, m2, red, wm, wn);
    if (wn == 0 && hl == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int row = m0 + lrow + rb * 32;
        if (row < M) st_dev2(reinterpret_cast<float2*>(a.partials) + (size_t)row * T2 + tn, make_float2(mu[rb], m2[rb]));
      }
    }
    wait_stores();
    __syncthreads();
    uint64_t* jw = a.joins + rowblk;
    if (t == 0) {
      // arrive; the last member advances the generation at once (every
      // member merges the partials itself, in member order)
      const uint64_t old = __hip_atomic_fetch_add(jw, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((uint32_t)old == (uint32_t)(T - 1))
        __hip_atomic_fetch_add(jw, (1ull << 32) - (uint64_t)T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      gen_sh = (uint32_t)(old >> 32);
    }
    __syncthreads();
    const uint32_t gen0 = gen_sh;
    return gen0;
  };

  // wait for the tile's row block, merge its statistics (every member, the
  // same way: member order, NP threads per row over contiguous runs, then
  // one thread per row over the runs), y = (u - mean) * rstd * gamma + beta,
  // stored
  auto finish = [&](f32x16(&acc)[RB][CB], int tile, uint32_t gen0) {
    const int rowblk = tile / T;
    const int tn = tile - rowblk * T;
    const int m0 = rowblk * BM, n0 = tn * BN;
    if (t == 0) wait_generation(a.joins + rowblk, gen0, a.err);
    __syncthreads();
    {
      constexpr int PER = 16;  // partials per thread per round trip (8 paired loads)
      const int r = t % BM, q = t / BM;
      const int per = ((T + NP - 1) / NP + 1) & ~1;  // even: runs start on a 16-byte pair
      const int kb = q * per, ke = min(T, kb + per);
      float cn = 0.0f, cm = 0.0f, c2 = 0.0f;
      // this tile's gamma and beta slices into LDS, in the same round trip
      for (int c = t; c < 2 * BN; c += THREADS) {
        const int cc = c < BN ? c : c - BN;
        const float v = bld4f(c < BN ? rGam : rBet, n0 + cc < N ? (uint32_t)(n0 + cc) * 4u : kOOB);
        vec[BN + c] = v;
      }
      if (m0 + r < M) {
        for (int k0 = kb; k0 < ke; k0 += PER) {
          u32x4 v[PER / 2];
#pragma unroll
          for (int k = 0; k < PER / 2; ++k)
            v[k] = bld16_dev(rP, k0 + 2 * k < ke ? (uint32_t)((m0 + r) * T2 + k0 + 2 * k) * 8u : kOOB);
#pragma unroll
          for (int k = 0; k < PER; ++k) {
            const int j = k0 + k;
            if (j < ke) {
              const float nj = (float)min(BN, N - j * BN);
              merge_ln(cn, cm, c2, nj, __uint_as_float(v[k >> 1][2 * (k & 1)]), __uint_as_float(v[k >> 1][2 * (k & 1) + 1]));
            }
          }
        }
      }
      parts[q * BM + r] = make_float4(cn, cm, c2, 0.0f);
      __syncthreads();
      if (t < BM) {
        float4 x = parts[t];
        for (int k = 1; k < NP; ++k) merge_ln(x.x, x.y, x.z, parts[k * BM + t].x, parts[k * BM + t].y, parts[k * BM + t].z);
        stat[t] = make_float2(x.y, rsqrtf(x.z / (float)N + a.eps));
      }
      __syncthreads();
    }
    float2 st[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) st[rb] = stat[lrow + rb * 32];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int cl = lcol + cb * 32 + 8 * h;
        const int col = n0 + cl;
        const bool ok = col < N;
        const float4 g0 = *reinterpret_cast<const float4*>(vec + BN + cl);
        const float4 g1 = *reinterpret_cast<const float4*>(vec + BN + cl + 4);
        const float4 b0 = *reinterpret_cast<const float4*>(vec + 2 * BN + cl);
        const float4 b1 = *reinterpret_cast<const float4*>(vec + 2 * BN + cl + 4);
        const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int row = m0 + lrow + rb * 32;
          float o[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = fmaf((acc[rb][cb][8 * h + e] - st[rb].x) * st[rb].y, gg[e], bb[e]);
          const u32x4 pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                            pack_bf16x2(o[6], o[7])};
          bst16(rY, (ok && row < M) ? (uint32_t)(row * N + col) * 2u : kOOB, pk);
        }
      }
    }
  };

  auto tile_at = [&](int r) { return round_tile(g, r, G, T, tiles, a.sw_a, a.sw_b); };
  if constexpr (PIPE) {
    // cur holds the tile waiting for its join while nxt's MainLoop runs
    f32x16 cur[RB][CB], nxt[RB][CB];
    int r = 0, tc = tile_at(0);
    uint32_t gc = produce(cur, tc, tile_at(1));
    for (;;) {
      const int tn1 = tile_at(r + 1);
      uint32_t gn = 0;
      if (tn1 >= 0) gn = produce(nxt, tn1, tile_at(r + 2));
      finish(cur, tc, gc);
      if (tn1 < 0) break;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) cur[rb][cb] = nxt[rb][cb];
      tc = tn1;
      gc = gn;
      ++r;
    }
  } else {
    f32x16 acc[RB][CB];
    for (int r = 0;; ++r) {
      const int tile = tile_at(r);
      if (tile < 0) break;
      const uint32_t gen0 = produce(acc, tile, -1);
      finish(acc, tile, gen0);
    }
  }
}

// GEMM + bias + residual + LayerNorm on large tiles: one workgroup of NWAVES
// waves per CU (the activation kernel's MainLoop and ring) computes ONE tile
// per launch; a launch covers a round of whole row blocks (every member of a
// row block resident at once), and the host launches one per round, so no
// register lives from one tile's epilogue into the next tile's MainLoop.  The
// tile's bias, gamma and beta slices reach LDS with three direct wave loads
// issued with the first stage.
//
// Epilogue, after the MainLoop:
//  * u = acc + R + bias, one row block of the lane's accumulators at a time
//    (up to three residual blocks in flight, the first issued behind the
//    last stage's MFMAs), and each block's lane statistics
//    (count, mean, M2 over the lane's valid columns) as soon as it is in;
//  * the lane pair and the column waves merged (tile statistics, one barrier);
//  * exchange with the other tiles of the row block through tagged slots
//    ([sass2mlir] "Counter-based mini-joins": one store publishes a value and
//    its tag, readers poll by tag): each member's (mean, M2) per row as two
//    64-bit {tag 1, value} slots, written once per launch.  Before its first
//    loads each member clears its own slots; it arrives on the row block's
//    join word after its MainLoop (the last member advances the generation),
//    and no member reads a slot before the generation has moved, so every
//    slot read holds 0 or this launch's value;
//  * every member merges the row block's partials in member order (the same
//    bits on every member), y = (u - mean) * rstd * gamma + beta, rounded to
//    bf16 into the idle ring and written as whole row segments with
//    non-temporal 16-byte stores.
template <int BM, int BN, int BK, int WGM, int NWAVES>
__global__ __launch_bounds__(NWAVES * 64, 1) void k_gemm_ln3(GemmArgs a) {
  using RG = Ring<BM, BN, BK, true, NWAVES>;
  constexpr int NS = 2;
  constexpr int THREADS = NWAVES * 64;
  constexpr int WGN = NWAVES / WGM;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int RB = WM / 32, CB = WN / 32;
  constexpr int NP = THREADS / BM;  // threads per row in the partial merge
  constexpr int C16 = BN * 2 / 16;  // 16-byte chunks per bf16 output row
  constexpr int RC0 = RG::STAGE_BYTES / (BN * 2);
  constexpr int RC = RC0 >= BM ? BM : (RC0 >= 128 ? 128 : (RC0 >= 64 ? 64 : 32));
  constexpr int MAXT = 16;          // tiles per row block whose slots the NP threads of a row take per batch
  static_assert(WM % 32 == 0 && WN % 32 == 0 && WGM * WGN == NWAVES && RB >= 2, "wave tile");
  static_assert(BM <= THREADS && THREADS % BM == 0 && NWAVES >= 3 && BN * 4 == 1024, "epilogue mapping");
  static_assert(RC0 >= 32 && BM % RC == 0 && (RC * C16) % THREADS == 0 && C16 >= 16, "output staging");
  static_assert((WGN * BM + THREADS) * 16 <= RG::STAGE_BYTES, "epilogue scratch in slot 0");
  __shared__ __align__(16) char s0[RG::STAGE_BYTES];
  __shared__ __align__(16) char s1[RG::STAGE_BYTES];
  __shared__ __align__(16) float vec[3][BN];  // bias | gamma | beta of the tile's columns (zero past N)
  __shared__ __align__(16) float2 stat[BM];   // (mean, rstd) per row
  float4* const red = reinterpret_cast<float4*>(s0);  // after the MainLoop: WGN x BM tile partials
  float4* const parts = red + WGN * BM;               // then NP x BM merged runs

  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int wm = w / WGN, wn = w % WGN;
  const int hl = lane >> 5, l32 = lane & 31;
  const int lrow = wm * WM + l32, lcol = wn * WN + 16 * hl;
  const int M = (int)a.M, N = (int)a.N;
  const int KT = (int)((a.K + BK - 1) / BK);
  const int T = a.tiles_n;
  // the launch's tiles [tile0, tile0 + G): with a swizzle (sw_a row x sw_b
  // column splits) each XCD takes a compact block of row blocks x column
  // tiles, so its L2 holds that block's A rows and W columns
  const int G = (int)gridDim.x;
  const int tile = a.tile0 + round_tile((int)xcd_local_id(blockIdx.x, (uint32_t)G), 0, G, T, a.tiles_m * T - a.tile0,
                                        a.sw_a, a.sw_b);
  if (tile < a.tile0 || tile >= a.tiles_m * T) return;
  const int rowblk = tile / T, tn = tile - rowblk * T;
  const int m0 = rowblk * BM, n0 = tn * BN;
  // tagged slots, member-major: {tag, mean} and {tag, M2} of row m0 + i of
  // member k at ((rowblk * T + k) * BM + i) * 2, so a wave's puts and takes
  // touch contiguous runs
  uint64_t* const slots = reinterpret_cast<uint64_t*>(a.partials) + (size_t)rowblk * T * BM * 2;
  const __amdgpu_buffer_rsrc_t rS = rsrc(slots, (uint32_t)(T * BM * 16));
  f32x16 acc[RB][CB];
  // residual: one row block of the lane's accumulators per fetch, RD in
  // flight; rows past M lie past the buffer's range and read zero, a chunk
  // past N reads the next row's values, which feed only columns past N,
  // never counted or stored
  constexpr int RD = RB >= 3 ? 3 : RB;
  const __amdgpu_buffer_rsrc_t rR = rsrc(a.R, a.R ? (uint32_t)(a.M * a.N * 2) : 0u);  // no residual: reads zero
  const uint32_t rbase = (uint32_t)((m0 + lrow) * N + n0 + lcol) * 2u;
  u32x4 rr[RD][CB][2];
  auto fetch = [&](auto rbc) {
    constexpr int rb = decltype(rbc)::value;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        rr[rb % RD][cb][h] = bld16(rR, rbase + (uint32_t)(32 * rb * N + 32 * cb + 8 * h) * 2u);
  };
  {
    const __amdgpu_buffer_rsrc_t rA = rsrc(a.A, (uint32_t)(a.M * a.K * 2));
    const __amdgpu_buffer_rsrc_t rB = rsrc(a.B, (uint32_t)(a.N * a.K * 2));
    const RG rg(a);
    char* const all_slots[2] = {s0, s1};
    zero_acc(acc);
    prologue_ns<BM, BN, BK, true, NWAVES, NS>(rg, rA, rB, all_slots, m0, n0, KT);
    if (w < 3) {
      const __amdgpu_buffer_rsrc_t rv = rsrc(w == 0 ? a.bias : w == 1 ? a.gamma : a.beta, (uint32_t)(a.N * 4));
      const int c = n0 + lane * 4;  // N % 8 == 0: a 16-byte chunk is wholly inside or past N
      g2l16(rv, &vec[w][0], c < N ? (uint32_t)c * 4u : kOOB);  // lane i fills bytes [16i, 16i + 16)
    }
    // clear this member's slots (the MainLoop's first wait completes the
    // stores, its barrier covers every thread's)
    if (t < BM && m0 + t < M) {
      slot_clear(slots + ((size_t)tn * BM + t) * 2);
      slot_clear(slots + ((size_t)tn * BM + t) * 2 + 1);
    }
    // the first residual block goes out behind the last stage's MFMAs
    main_loop_ns<BM, BN, BK, true, RB, CB, NWAVES, NS>(rg, rA, rB, all_slots, m0, n0, false, 0, 0, acc, KT, wm, wn,
                                                        [&](int st) {
                                                          if (st == KT - 1) fetch(IntC<0>{});
                                                        });
  }
  // arrive on the row block's launch join (every member's slots are clear by now)
  uint64_t* const jw = a.joins + rowblk;
  uint64_t jold = 0;
  if (t == 0) jold = join_arrive(jw, (uint32_t)T);

  // ---- u = acc + R + bias and the lane statistics, one row block of the
  // lane's accumulators at a time as its residual block lands
  const bool full = n0 + BN <= N;  // uniform: every column of the tile is valid
  int nvalid = 0;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int h = 0; h < 2; ++h) nvalid += (n0 + lcol + cb * 32 + 8 * h < N) ? 8 : 0;
  float n_[RB], mu[RB], m2[RB];
  {
    auto block = [&](auto rbc) {
      constexpr int rb = decltype(rbc)::value;
      float sum = 0.0f;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int cl = lcol + cb * 32 + 8 * h;
          const float4 b0 = *reinterpret_cast<const float4*>(&vec[0][cl]);
          const float4 b1 = *reinterpret_cast<const float4*>(&vec[0][cl + 4]);
          const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
          const bool ok = full || n0 + cl < N;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t wv = rr[rb % RD][cb][h][e >> 1];
            const float u = acc[rb][cb][8 * h + e] + ((e & 1) ? bf16_hi(wv) : bf16_lo(wv)) + bv[e];
            acc[rb][cb][8 * h + e] = u;
            sum += ok ? u : 0.0f;
          }
        }
      const float mean = nvalid > 0 ? sum / (float)nvalid : 0.0f;
      float q2 = 0.0f;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const float d = (full || n0 + lcol + cb * 32 + (q & 8) < N) ? acc[rb][cb][q] - mean : 0.0f;
          q2 = fmaf(d, d, q2);
        }
      n_[rb] = (float)nvalid;
      mu[rb] = mean;
      m2[rb] = q2;
    };
    for_each_c([&](auto qc) { fetch(IntC<decltype(qc)::value + 1>{}); }, std::make_integer_sequence<int, RD - 1>{});
    __syncthreads();  // every wave is done with the ring (slot 0 becomes the epilogue scratch); vec is in
    for_each_c(
        [&](auto qc) {
          constexpr int Q = decltype(qc)::value;
          // block Q is in; the blocks after it (at most RD - 1) may still fly
          constexpr int after = (RB - 1 - Q) < (RD - 1) ? (RB - 1 - Q) : (RD - 1);
          wait_vm<after * CB * 2>();
          block(IntC<Q>{});
          if constexpr (Q + RD < RB) fetch(IntC<Q + RD>{});
        },
        std::make_integer_sequence<int, RB>{});
  }
  tile_merge_ln<BM, WGN, RB>(n_, mu, m2, red, wm, wn);
  if (wn == 0 && hl == 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = m0 + lrow + rb * 32;
      if (row < M) {
        slot_put(slots + ((size_t)tn * BM + row - m0) * 2, 1u, mu[rb]);
        slot_put(slots + ((size_t)tn * BM + row - m0) * 2 + 1, 1u, m2[rb]);
      }
    }
  }
  if (t == 0) join_await(jw, jold, (uint32_t)T, a.err);  // every member's slots were cleared
  __syncthreads();

  // ---- the row block's statistics: NP threads per row take contiguous runs
  // of members' slots (all in flight at once, re-polled until tagged), merge
  // them in member order, then one thread per row merges the runs
  {
    const int rw = t % BM, q = t / BM;
    const int per = (T + NP - 1) / NP;
    const int kb = q * per, ke = min(T, kb + per);
    float cn = 0.0f, cm = 0.0f, c2 = 0.0f;
    if (m0 + rw < M) {
      for (int k0 = kb; k0 < ke; k0 += MAXT / NP) {
        const int kn = min(ke - k0, MAXT / NP);
        float mv[MAXT / NP], qv[MAXT / NP];
        uint64_t pending = kn >= 64 ? ~0ull : ((1ull << kn) - 1);
        for (uint32_t it = 0; pending != 0 && it < kSpinCap; ++it) {
          // every poll's loads in flight together (no load sits in a branch
          // of its own, which would wait out each one); a member past the
          // batch re-reads member k0 and is ignored
          // a member's two slots of a row are one 16-byte pair: one device-scope
          // load reads both (each 8-byte half is one store's word)
          u32x4 xv[MAXT / NP];
#pragma unroll
          for (int k = 0; k < MAXT / NP; ++k)
            xv[k] = bld16_dev(rS, (uint32_t)(((k < kn ? k0 + k : k0) * BM + rw) * 16));
#pragma unroll
          for (int k = 0; k < MAXT / NP; ++k)
            if ((pending >> k & 1) && xv[k][1] == 1u && xv[k][3] == 1u) {
              mv[k] = __uint_as_float(xv[k][0]);
              qv[k] = __uint_as_float(xv[k][2]);
              pending &= ~(1ull << k);
            }
          if (pending != 0) __builtin_amdgcn_s_sleep(2);
        }
        if (pending != 0) __hip_atomic_fetch_or(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int k = 0; k < MAXT / NP; ++k)
          if (k < kn && !(pending >> k & 1)) merge_ln(cn, cm, c2, (float)min(BN, N - (k0 + k) * BN), mv[k], qv[k]);
      }
    }
    parts[q * BM + rw] = make_float4(cn, cm, c2, 0.0f);
    __syncthreads();
    if (t < BM) {
      float4 x = parts[t];
      for (int k = 1; k < NP; ++k) merge_ln(x.x, x.y, x.z, parts[k * BM + t].x, parts[k * BM + t].y, parts[k * BM + t].z);
      stat[t] = make_float2(x.y, rsqrtf(x.z / (float)N + a.eps));
    }
    __syncthreads();
  }

  // ---- y = (u - mean) * rstd * gamma + beta, bf16, staged through slot 1 in
  // chunks of RC whole rows, written as non-temporal 16-byte row segments
  float2 st[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) st[rb] = stat[lrow + rb * 32];
  uint16_t* const stg = reinterpret_cast<uint16_t*>(s1);
#pragma unroll 1
  for (int qc = 0; qc < BM / RC; ++qc) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int cl = lcol + cb * 32 + 8 * h;
        const float4 g0 = *reinterpret_cast<const float4*>(&vec[1][cl]);
        const float4 g1 = *reinterpret_cast<const float4*>(&vec[1][cl + 4]);
        const float4 b0 = *reinterpret_cast<const float4*>(&vec[2][cl]);
        const float4 b1 = *reinterpret_cast<const float4*>(&vec[2][cl + 4]);
        const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int rl = wm * WM + rb * 32;  // the wave's 32 rows of this block (uniform)
          if (rl / RC != qc) continue;
          const int rr = rl - qc * RC + l32;
          float o[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = fmaf((acc[rb][cb][8 * h + e] - st[rb].x) * st[rb].y, gg[e], bb[e]);
          const u32x4 pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                            pack_bf16x2(o[6], o[7])};
          *reinterpret_cast<u32x4*>(stg + rr * BN + 8 * eswz(rr, cl / 8)) = pk;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < RC * C16 / THREADS; ++j) {
      const int id = j * THREADS + t;
      const int rr = id / C16, c = id % C16;
      const int row = m0 + qc * RC + rr, col = n0 + 8 * c;
      if (row < M && col < N)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(stg + rr * BN + 8 * eswz(rr, c)),
                                    reinterpret_cast<u32x4*>(a.Y + (int64_t)row * N + col));
    }
    __syncthreads();
  }
}

// GEMM + unary activation on large tiles, one workgroup of NWAVES waves per
// CU walking tiles XCD-locally.  The tiles are independent (each output
// element has one owner), so there is no join; while a tile's epilogue runs,
// the first NS-1 stages of the workgroup's next tile are already in flight.
// The tile's bias slice goes to LDS with one direct load issued before the
// MainLoop (double-buffered by tile parity, so the next tile's slice never
// overwrites one still being read); its completion is covered by the
// MainLoop's own waits, which retire every load issued before the last stage.
// Lane (rb, cb) results are 16 consecutive columns of one row; each lane
// writes its 32-byte row segment as two 16-byte stores (L2 merges the halves).
template <int BM, int BN, int BK, int WGM, int NWAVES, int NS>
__global__ __launch_bounds__(NWAVES * 64, 1) void k_gemm_act2(GemmArgs a) {
  using RG = Ring<BM, BN, BK, true, NWAVES>;
  constexpr int WGN = NWAVES / WGM;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int RB = WM / 32, CB = WN / 32;
  static_assert(WM % 32 == 0 && WN % 32 == 0 && WGM * WGN == NWAVES, "wave tile");
  static_assert(NS >= 2 && NS <= 4, "ring depth");
  static_assert(BN * 4 <= 64 * 16, "one wave load carries the bias slice");
  constexpr int THREADS = NWAVES * 64;
  constexpr int C16 = BN * 2 / 16;  // 16-byte chunks per bf16 output row
  // output rows staged per chunk: the largest power of two (at most BM) whose rows fit one slot
  constexpr int RC0 = RG::STAGE_BYTES / (BN * 2);
  constexpr int RC = RC0 >= BM ? BM : (RC0 >= 128 ? 128 : (RC0 >= 64 ? 64 : 32));
  static_assert(RC0 >= 32 && BM % RC == 0 && (RC * C16) % THREADS == 0 && C16 >= 16, "output staging");
  __shared__ __align__(16) char s0[RG::STAGE_BYTES];
  __shared__ __align__(16) char s1[RG::STAGE_BYTES];
  __shared__ __align__(16) char s2[NS > 2 ? RG::STAGE_BYTES : 16];
  __shared__ __align__(16) char s3[NS > 3 ? RG::STAGE_BYTES : 16];
  __shared__ __align__(16) float bias_sl[2][BN];

  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int wm = w / WGN, wn = w % WGN;
  const int hl = lane >> 5, l32 = lane & 31;
  const int M = (int)a.M, N = (int)a.N;
  const int KT = (int)((a.K + BK - 1) / BK);
  const int G = (int)gridDim.x;
  const int g = (int)xcd_local_id(blockIdx.x, (uint32_t)G);
  const int T = a.tiles_n;
  const int tiles = a.tiles_m * T;
  if (g >= tiles) return;
  const __amdgpu_buffer_rsrc_t rA = rsrc(a.A, (uint32_t)(a.M * a.K * 2));
  const __amdgpu_buffer_rsrc_t rB = rsrc(a.B, (uint32_t)(a.N * a.K * 2));
  const __amdgpu_buffer_rsrc_t rBias = rsrc(a.bias, a.bias ? (uint32_t)(a.N * 4) : 0u);  // no bias: reads zero
  const RG rg(a);
  char* const all_slots[4] = {s0, s1, s2, s3};
  char* sl[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) sl[q] = all_slots[q];
  bool staged = false;  // the tile's first stages are already in the ring
  int par = 0;

  for (int tile = g; tile < tiles; tile += G, par ^= 1) {
    const int next = tile + G < tiles ? tile + G : -1;
    const int m0 = (tile / T) * BM, n0 = (tile % T) * BN;
    f32x16 acc[RB][CB];
    zero_acc(acc);
    if (!staged) {
      __syncthreads();  // every wave is done with the ring
      prologue_ns<BM, BN, BK, true, NWAVES, NS>(rg, rA, rB, sl, m0, n0, KT);
    }
    if (w == 0 && lane * 4 < BN) {
      const int c = n0 + lane * 4;  // N % 8 == 0: a chunk is wholly inside or past N
      g2l16(rBias, bias_sl[par], c < N ? (uint32_t)c * 4u : kOOB);  // lane i fills bytes [16i, 16i + 16)
    }
    const bool pre = next >= 0 && KT % NS == 0;
    main_loop_ns<BM, BN, BK, true, RB, CB, NWAVES, NS>(rg, rA, rB, sl, m0, n0, pre, (next / T) * BM,
                                                       (next % T) * BN, acc, KT, wm, wn);
    staged = pre;
    const float* bsl = bias_sl[par];
    // The results leave through the ring's last slot (free here: the next
    // tile's prefetch fills the others) in chunks of RC whole rows, then as
    // non-temporal 16-byte stores of whole row segments: one write per
    // output line instead of two half-line writes from the lane layout.
    uint16_t* const stg = reinterpret_cast<uint16_t*>(sl[NS - 1]);
    __syncthreads();  // every wave is done reading the last slot
    auto finish = [&](auto actc) {
      constexpr int ACT = decltype(actc)::value;
#pragma unroll 1
      for (int q = 0; q < BM / RC; ++q) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int cl0 = wn * WN + cb * 32 + 16 * hl;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float4 b0 = *reinterpret_cast<const float4*>(bsl + cl0 + 8 * h);
            const float4 b1 = *reinterpret_cast<const float4*>(bsl + cl0 + 8 * h + 4);
            const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
              const int rl = wm * WM + rb * 32;  // the wave's 32 rows of this block (uniform)
              if (rl / RC != q) continue;
              const int rr = rl - q * RC + l32;
              float o[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) o[e] = act_fn<ACT>(acc[rb][cb][8 * h + e] + bb[e]);
              const u32x4 pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                                pack_bf16x2(o[6], o[7])};
              *reinterpret_cast<u32x4*>(stg + rr * BN + 8 * eswz(rr, cl0 / 8 + h)) = pk;
            }
          }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < RC * C16 / THREADS; ++j) {
          const int id = j * THREADS + t;
          const int rr = id / C16, c = id % C16;
          const int row = m0 + q * RC + rr, col = n0 + 8 * c;
          if (row < M && col < N)
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(stg + rr * BN + 8 * eswz(rr, c)),
                                        reinterpret_cast<u32x4*>(a.Y + (int64_t)row * N + col));
        }
        __syncthreads();
      }
    };
    switch (a.act) {
      case kActRelu: finish(IntC<kActRelu>{}); break;
      case kActGeluTanh: finish(IntC<kActGeluTanh>{}); break;
      case kActSilu: finish(IntC<kActSilu>{}); break;
      case kActSquare: finish(IntC<kActSquare>{}); break;
      case kActRsqrt: finish(IntC<kActRsqrt>{}); break;
      default: finish(IntC<kActNone>{}); break;
    }
  }
}

// ---------------------------------------------------------------- dispatch

struct TileCfg {
  int bm, bn, bk;
};

// Tile configurations (id -> shape); the launch lists below must match.
// Round-based kernel (plain GEMM, and the fused epilogues' schedule 0):
static const TileCfg kCfgs[] = {
    {256, 256, 64},  // 0: 2x2 waves of 128x128, 2-slot ring 128 KB, 1 WG/CU
    {256, 128, 64},  // 1: 2x2 waves of 128x64, 2-stage ring 96 KB, 1 WG/CU
    {128, 256, 64},  // 2: 2x2 waves of 64x128, 2-stage ring 96 KB, 1 WG/CU
    {128, 128, 64},  // 3: 2x2 waves of 64x64, 2-stage ring 64 KB, 2 WG/CU
    {64, 512, 64},   // 4: 1x4 waves of 64x128, 2-stage ring 144 KB, 1 WG/CU
    {128, 128, 32},  // 5: 2x2 waves of 64x64, 2-stage ring 32 KB, 2 WG/CU
};
// GEMM + LN with overlapped joins (k_gemm_ln2):
static const TileCfg kLnCfgs[] = {
    {256, 256, 32},  // 0: 8 waves of 128x64, 4-slot ring 128 KB, 1 WG/CU, one tile at a time
    {256, 128, 32},  // 1: 2x2 waves of 128x64, 4-slot ring 96 KB, 1 WG/CU, pipelined
    {128, 256, 32},  // 2: 2x2 waves of 64x128, 4-slot ring 96 KB, 1 WG/CU, pipelined
    {128, 128, 64},  // 3: 2x2 waves of 64x64, 2-slot ring 64 KB, 2 WG/CU, pipelined
    {128, 128, 64},  // 4: 2x2 waves of 64x64, 4-slot ring 128 KB, 1 WG/CU, pipelined
    {128, 128, 32},  // 5: 2x2 waves of 64x64, 4-slot ring 64 KB, 2 WG/CU, pipelined
    {128, 128, 32},  // 6: 2x2 waves of 64x64, 2-slot ring 32 KB, 2 WG/CU, pipelined
    {256, 256, 64},  // 7: 8 waves of 128x64, 2-slot ring 128 KB, 1 WG/CU, one tile at a time, residual streamed in
};

static const TileCfg kActCfgs[] = {
    {256, 256, 64},  // 0: 8 waves of 128x64, 2-slot ring, 1 WG/CU
    {256, 256, 32},  // 1: 8 waves of 128x64, 4-slot ring, 1 WG/CU
    {256, 128, 64},  // 2: 8 waves of 64x64, 2-slot ring, 1 WG/CU
    {256, 128, 64},  // 3: 8 waves of 64x64, 3-slot ring, 1 WG/CU
};

bool gemm_tile_config(int epi, int algo, int cfg, int* bm, int* bn, int* bk) {
  if (epi == kEpiAct && algo == 1) {
    if (cfg < 0 || cfg >= (int)(sizeof(kActCfgs) / sizeof(kActCfgs[0]))) return false;
    *bm = kActCfgs[cfg].bm;
    *bn = kActCfgs[cfg].bn;
    *bk = kActCfgs[cfg].bk;
    return true;
  }
  const bool ln2 = epi == kEpiLN && algo == 1;
  const TileCfg* t = ln2 ? kLnCfgs : kCfgs;
  const int n = ln2 ? (int)(sizeof(kLnCfgs) / sizeof(kLnCfgs[0])) : (int)(sizeof(kCfgs) / sizeof(kCfgs[0]));
  if (cfg < 0 || cfg >= n) return false;
  // the round-based epilogue kernels exist for tiles of at most 128 x 256
  if (!ln2 && epi != kEpiStoreF32 && t[cfg].bm * t[cfg].bn > 128 * 256) return false;
  *bm = t[cfg].bm;
  *bn = t[cfg].bn;
  *bk = t[cfg].bk;
  return true;
}

template <int EPI, bool NN>
static hipError_t launch_gemm_t(const GemmPlan& pl, const GemmArgs& a, hipStream_t st, int* occ) {
#define CF_GEMM(CFG, BM, BN, BK, WGM, STG, MINB)                                                        \
  if constexpr (EPI == kEpiStoreF32 || BM * BN <= 128 * 256)                                            \
  if (pl.cfg == CFG) {                                                                                  \
    auto kfn = k_gemm<EPI, NN, BM, BN, BK, WGM, STG, MINB>;                                              \
    if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, kfn, kThreads, 0);                \
    hipLaunchKernelGGL(kfn, dim3(pl.grid), dim3(kThreads), 0, st, a);                                   \
    return hipGetLastError();                                                                           \
  }
  CF_GEMM(0, 256, 256, 64, 2, 2, 1)
  CF_GEMM(1, 256, 128, 64, 2, 2, 1)
  CF_GEMM(2, 128, 256, 64, 2, 2, 1)
  CF_GEMM(3, 128, 128, 64, 2, 2, 2)
  CF_GEMM(4, 64, 512, 64, 1, 2, 1)
  CF_GEMM(5, 128, 128, 32, 2, 2, 2)
#undef CF_GEMM
  return hipErrorInvalidConfiguration;
}

template <int EPI>
static hipError_t launch_gemm_overlap(const GemmPlan& pl, const GemmArgs& a, hipStream_t st, int* occ) {
  auto go = [&](auto kfn, int threads) -> hipError_t {
    if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, kfn, threads, 0);
    hipLaunchKernelGGL(kfn, dim3(pl.grid), dim3(threads), 0, st, a);
    return hipGetLastError();
  };
  if constexpr (EPI == kEpiLN) {
    switch (pl.cfg) {
      case 0: return go(k_gemm_ln2<256, 256, 32, 2, 1, 8, false, 4>, 512);  // 8 waves of 128x64, one tile per round
      case 1: return go(k_gemm_ln2<256, 128, 32, 2, 1, 4, true, 4>, 256);
      case 2: return go(k_gemm_ln2<128, 256, 32, 2, 1, 4, true, 4>, 256);
      case 3: return go(k_gemm_ln2<128, 128, 64, 2, 2, 4, true, 2>, 256);
      case 4: return go(k_gemm_ln2<128, 128, 64, 2, 1, 4, true, 4>, 256);
      case 5: return go(k_gemm_ln2<128, 128, 32, 2, 2, 4, true, 4>, 256);
      case 6: return go(k_gemm_ln2<128, 128, 32, 2, 2, 4, true, 2>, 256);
      case 7: {  // 8 waves of 128x64, one tile per workgroup: one launch per round
        auto kfn = k_gemm_ln3<256, 256, 64, 2, 8>;
        if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, kfn, 512, 0);
        const int tiles = a.tiles_m * a.tiles_n;
        for (int t0 = 0; t0 < tiles; t0 += pl.grid) {
          GemmArgs ar = a;
          ar.tile0 = t0;
          const int g = std::min(pl.grid, tiles - t0);
          if (g != pl.grid) ar.sw_a = ar.sw_b = 0;  // the XCD split is sized for a full round
          hipLaunchKernelGGL(kfn, dim3(g), dim3(512), 0, st, ar);
          const hipError_t e = hipGetLastError();
          if (e != hipSuccess) return e;
        }
        return hipSuccess;
      }
    }
  } else {
    switch (pl.cfg) {
      case 1: return go(k_gemm_sm2<256, 128, 64, 2, 1>, 256);
      case 2: return go(k_gemm_sm2<128, 256, 64, 2, 1>, 256);
      case 3: return go(k_gemm_sm2<128, 128, 64, 2, 2>, 256);
      case 4: return go(k_gemm_sm2<64, 512, 64, 1, 1>, 256);
      case 5: return go(k_gemm_sm2<128, 128, 32, 2, 2>, 256);
    }
  }
  return hipErrorInvalidConfiguration;
}

static hipError_t gemm_dispatch(int epi, const GemmPlan& pl, const GemmArgs& a, hipStream_t st, int* occ) {
  if (epi == kEpiLN) {
    if (!pl.nn) return hipErrorInvalidConfiguration;
    return pl.algo == 1 ? launch_gemm_overlap<kEpiLN>(pl, a, st, occ) : launch_gemm_t<kEpiLN, true>(pl, a, st, occ);
  }
  if (epi == kEpiAct) {
    if (!pl.nn) return hipErrorInvalidConfiguration;
    if (pl.algo == 0) return launch_gemm_t<kEpiAct, true>(pl, a, st, occ);
    auto go = [&](auto kfn, int threads) -> hipError_t {
      if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, kfn, threads, 0);
      hipLaunchKernelGGL(kfn, dim3(pl.grid), dim3(threads), 0, st, a);
      return hipGetLastError();
    };
    switch (pl.cfg) {
      case 0: return go(k_gemm_act2<256, 256, 64, 2, 8, 2>, 512);  // 8 waves of 128x64, 2-slot ring 128 KB
      case 1: return go(k_gemm_act2<256, 256, 32, 2, 8, 4>, 512);  // 8 waves of 128x64, 4-slot ring 128 KB
      case 2: return go(k_gemm_act2<256, 128, 64, 4, 8, 2>, 512);  // 8 waves of 64x64, 2-slot ring 96 KB
      case 3: return go(k_gemm_act2<256, 128, 64, 4, 8, 3>, 512);  // 8 waves of 64x64, 3-slot ring 144 KB
    }
    return hipErrorInvalidConfiguration;
  }
  if (epi == kEpiSoftmaxGemm) {
    if (pl.nn || pl.algo != 2) return hipErrorInvalidConfiguration;
    auto kfn = pl.bk <= 32 ? k_gemm_b2b<2, 4> : (pl.bk <= 64 ? k_gemm_b2b<4, 4> : k_gemm_b2b<8, 4>);
    if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, kfn, kB2bThreads, 0);
    hipLaunchKernelGGL(kfn, dim3(pl.grid), dim3(kB2bThreads), 0, st, a);
    return hipGetLastError();
  }
  if (epi == kEpiSoftmax) {
    if (pl.nn) return hipErrorInvalidConfiguration;
    if (pl.algo == 2) {
      auto kfn = pl.bk <= 32 ? k_gemm_sm3<2, 2> : (pl.bk <= 64 ? k_gemm_sm3<4, 2> : k_gemm_sm3<8, 2>);
      if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, kfn, kThreads, 0);
      hipLaunchKernelGGL(kfn, dim3(pl.grid), dim3(kThreads), 0, st, a);
      return hipGetLastError();
    }
    return pl.algo == 1 ? launch_gemm_overlap<kEpiSoftmax>(pl, a, st, occ)
                        : launch_gemm_t<kEpiSoftmax, false>(pl, a, st, occ);
  }
  return pl.nn ? launch_gemm_t<kEpiStoreF32, true>(pl, a, st, occ) : launch_gemm_t<kEpiStoreF32, false>(pl, a, st, occ);
}

hipError_t launch_gemm(int epi, const GemmPlan& pl, const GemmArgs& a, hipStream_t st) {
  return gemm_dispatch(epi, pl, a, st, nullptr);
}

hipError_t gemm_occupancy(int epi, const GemmPlan& pl, int* per_cu) {
  return gemm_dispatch(epi, pl, GemmArgs{}, nullptr, per_cu);
}

}  // namespace cf
