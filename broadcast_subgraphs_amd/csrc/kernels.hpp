// Host-visible launch interfaces of the kernels (internal to libcf.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dev.hpp"

namespace cf {

enum RowOp { kSoftmax = 0, kLayerNorm = 1, kPowSoftmax = 2, kLayerNormAffine = 3, kRmsNorm = 4 };
// LayerNorm (with or without its affine map) and RMSNorm: one reduction
// family; RMSNorm is the LayerNorm stage chain with the mean held at 0.
constexpr bool is_norm(int op) { return op == kLayerNorm || op == kLayerNormAffine || op == kRmsNorm; }

struct RowArgs {
  const float* x;
  float* y;
  float* y_pre;     // pow-softmax only, nullable
  const float* v;   // pow-softmax only
  const float* gamma;  // affine LayerNorm: [cols]; RMSNorm: [cols] or null (gain 1)
  const float* beta;   // affine LayerNorm: [cols]
  float p;
  float eps;
  int64_t rows;
  int64_t cols;
  uint32_t* err;    // workspace error word
  uint64_t* joins;  // split plans: one join word per group of S workgroups
  uint64_t* slots;  // split plans: groups * 4 * S tagged slots ([parity][field][member])
  int S;            // workgroups per row (split plans), at most kMaxSplit
  int64_t slice;    // columns per member (split plans)
};

// Most workgroups one row may be split over (the members' partials of a row
// sit in LDS while they are merged).
constexpr int kMaxSplit = 256;

struct RowPlan {
  int block = 256;  // lanes per workgroup (256; 512 or 1024 for one wide row per workgroup)
  int w = 4;      // floats per fragment (4 or 1)
  int lpr = 256;  // lanes per row (in-workgroup plans)
  int nv = 1;     // fragments per lane per row
  int rpi = 1;    // rows in flight per lane
  int split = 1;  // workgroups per row (>1: split plan)
  int64_t slice = 0;
  int grid = 1;
  int occupancy = 0;  // resident workgroups per CU (split plans)
};

hipError_t launch_rows(int op, const RowPlan& pl, const RowArgs& a, hipStream_t st);
hipError_t rows_split_occupancy(int op, const RowPlan& pl, int* per_cu);

// ----------------------------------------------------------------- GEMM
enum GemmEpi { kEpiStoreF32 = 0, kEpiLN = 1, kEpiSoftmax = 2, kEpiSoftmaxGemm = 3, kEpiAct = 4 };

// unary activations of the activation epilogue (the same ids as the C-ABI's CF_ACT_*)
enum ActId { kActNone = 0, kActRelu = 1, kActGeluTanh = 2, kActSilu = 3, kActSquare = 4, kActRsqrt = 5 };

// Back-to-back GEMM kernel shape: 256-row strips of 64-key tiles, one 8-wave
// workgroup per CU, the reduction dimension up to 128.
constexpr int kB2bBM = 256, kB2bBN = 64, kB2bBK = 128, kB2bWaves = 8, kB2bThreads = kB2bWaves * 64;

struct GemmArgs {
  const uint16_t* A;   // [M x K] bf16 (GEMM left operand; Q for softmax)
  const uint16_t* B;   // NN: W [K x N]; NT: K [N x K] (bf16)
  const float* bias;   // LN: [N]
  const uint16_t* R;   // LN: [M x N] bf16, nullable
  const float* gamma;  // LN: [N]
  const float* beta;   // LN: [N]
  float eps;
  float scale;         // softmax: multiplies the accumulator
  uint16_t* Y;         // bf16 [M x N] output (LN, softmax)
  float* Z;            // fp32 [M x N] output (plain GEMM)
  int64_t M, N, K;
  int tiles_n;         // column tiles per row group = ceil(N / BN)
  int tiles_m;
  uint32_t* err;
  uint64_t* joins;     // one join word per group of tiles_n workgroups
  float* partials;     // M * tiles_n * 4 floats
  float* finals;       // M * 2 floats: the leader's per-row results (strip softmax: max + log2(sum), unused)
  int agg_leader;      // 0: every member reads all partials; 1: last arriver combines
  int strips;          // strip softmax: strips per row block
  int sw_a, sw_b;      // LN: per-round tile blocks per XCD (sw_a row x sw_b column splits; 0 = linear)
  const uint16_t* V;   // softmax-GEMM: second operand [N x Dv] bf16 (Y is then O [M x Dv])
  int64_t Dv;
  float* opart;        // softmax-GEMM: per-strip partial outputs, M * strips * 128 bf16, then (max, sum) pairs
  int act;             // activation epilogue: ActId (bias nullable)
  int tile0;           // one-tile-per-workgroup kernels launched per round: the round's first tile
};

struct GemmPlan {
  int cfg = 0;        // tile configuration id
  int bm = 256, bn = 256, bk = 64;
  int nn = 1;         // 1: B is [K x N]; 0: B is [N x K]
  int grid = 0;
  int occupancy = 0;  // resident workgroups per CU
  int tiles = 0;
  int rounds = 0;
  bool leader = false;  // last-arriver aggregation (else every member reads all partials)
  int algo = 1;         // fused epilogues: 0 = one join per round, 1 = joins overlapped with MainLoops,
                        // 2 = softmax by strips (reduction dimension <= 128)
  int strips = 1;       // algo 2: strips per row block
  int sw_a = 0, sw_b = 0;  // algo 1 LN: XCD tile-block split of each round (0 = linear order)
};

// Tiles one workgroup may take per sweep in the two-sweep softmax epilogue
// (the generation each tile's row block arrived in is logged in LDS).
constexpr int kMaxRounds = 256;

hipError_t launch_gemm(int epi, const GemmPlan& pl, const GemmArgs& a, hipStream_t st);
hipError_t gemm_occupancy(int epi, const GemmPlan& pl, int* per_cu);
bool gemm_tile_config(int epi, int algo, int cfg, int* bm, int* bn, int* bk);

// ----------------------------------------------------------- unfused ops
hipError_t u_rowreduce(const float* x, float* out, int64_t rows, int64_t cols, int is_max, hipStream_t st);
// y = x (op) c[row]  for op: 0 sub, 1 div, 2 mul, 3 add
hipError_t u_bcast_col(const float* x, const float* c, float* y, int64_t rows, int64_t cols, int op, hipStream_t st);
// y = x (op) r[col]  for op: 2 mul, 3 add
hipError_t u_bcast_row(const float* x, const float* r, float* y, int64_t rows, int64_t cols, int op, hipStream_t st);
// y = f(x) elementwise: 0 exp, 1 square, 2 pow(x, p), 3 rsqrt(x/n + eps) , 4 scale(x, p),
// 5 relu, 6 tanh-form gelu, 7 silu, 8 rsqrt(x)
hipError_t u_map(const float* x, float* y, int64_t n, int op, float p, float q, hipStream_t st);
hipError_t u_add_bf16(const float* x, const uint16_t* r, float* y, int64_t n, hipStream_t st);
hipError_t u_cast_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t st);
hipError_t u_fill(float* p, int64_t n, float v, hipStream_t st);
hipError_t u_copy(const float* s, float* d, int64_t n, hipStream_t st);

}  // namespace cf
