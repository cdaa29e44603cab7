// C-ABI entry points: argument validation, planning and launch.
//
// The planner is a pure function of the shape and the device's properties,
// with no autotuning ([AStitch] "Adaptive thread mapping": the mapping is
// chosen just in time from the real shapes).  Rows that fit a workgroup are
// packed (many short rows per workgroup, several rows in flight per lane) or
// mapped one per workgroup; rows that do not fit are split across workgroups
// that aggregate through global memory.  Any plan whose workgroups wait on
// each other is sized to the grid the device keeps resident at once
// ([AStitch] "What it costs"), or refused with CF_EOCCUPANCY.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/cf.h"
#include "kernels.hpp"

using namespace cf;

namespace {

thread_local std::string g_last_plan;

struct DevInfo {
  int cus = 0;
  bool ok = false;
};
constexpr int kMaxDev = 64;
DevInfo g_dev[kMaxDev];
std::once_flag g_dev_once[kMaxDev];

cf_status dev_info(DevInfo** out) {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= kMaxDev) return CF_EHIP;
  std::call_once(g_dev_once[d], [d] {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, d) == hipSuccess) {
      g_dev[d].cus = p.multiProcessorCount;
      g_dev[d].ok = true;
    }
  });
  if (!g_dev[d].ok) return CF_EHIP;
  *out = &g_dev[d];
  return CF_OK;
}

long env_int(const char* name, long dflt) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  return strtol(s, nullptr, 10);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int pow2ceil(int64_t v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

// Workspace layout, the same for every plan of every op:
//   [0, 256)                      header (u32 error word at offset 0)
//   [256, 256 + 8 * kMaxJoins)    join words, one per group of cooperating
//                                 workgroups (group membership is fixed for a
//                                 launch, so a join word serves every round)
//   [kPartialsOff, ...)           per-row partials
// Because the join region is fixed, one op's partials never overwrite another
// op's join words, and every completed join leaves its count at 0: a workspace
// can be reused by any later call of any op.
constexpr size_t kHeader = 256;
constexpr int64_t kMaxJoins = 16384;
constexpr size_t kPartialsOff = kHeader + kMaxJoins * sizeof(uint64_t);

struct WsLayout {
  size_t joins_off = 0, partials_off = 0, total = 0;
};

WsLayout ws_layout(int64_t npartial_floats) {
  WsLayout L;
  L.joins_off = kHeader;
  L.partials_off = kPartialsOff;
  L.total = align_up(kPartialsOff + (size_t)npartial_floats * sizeof(float), 256);
  return L;
}

// ------------------------------------------------------------ row planning

cf_status plan_rows(int op, int64_t rows, int64_t cols, bool vec_ok, RowPlan* pl) {
  DevInfo* di = nullptr;
  cf_status s = dev_info(&di);
  if (s != CF_OK) return s;
  RowPlan p;
  p.w = (vec_ok && cols % 4 == 0) ? 4 : 1;
  const int64_t nvec = (cols + p.w - 1) / p.w;
  const long force_split = env_int("CF_FORCE_SPLIT", 0);
  const long force_wide = env_int("CF_FORCE_WIDE", -1);  // 1: one wide row per workgroup, 0: never
  if (nvec <= 64 && force_split <= 1) {
    p.lpr = (int)std::max<int64_t>(4, pow2ceil(nvec));
    p.nv = 1;
    p.rpi = (int)env_int("CF_FORCE_RPI", p.lpr <= 16 ? 2 : 1);
  } else if (nvec <= 256 * 16 && force_split <= 1) {
    p.lpr = 256;
    p.nv = pow2ceil((nvec + 255) / 256);
    p.rpi = 1;
  } else if (force_split <= 1 && force_wide != 0 && nvec <= 1024 * (op == kLayerNormAffine && p.w == 4 ? 4 : 8)) {
    // wide rows: one row per workgroup of 1024 lanes holds the whole row
    // (<= 8 fragments per lane), so no cross-workgroup exchange is needed,
    // whatever the row count (measured on MI355X against two members per
    // row: 512 x 32768 23.5 against 34.6 us, 4000 x 20000 110.3 against
    // 133.2 us, 300 x 20000 10.1 against 13.5 us).
    // Affine LayerNorm on 16-byte fragments takes at most 4: with its gain
    // and bias fragments, 8 exceed the registers a 1024-lane workgroup's
    // waves have (measured: spills cost it 15 us on 64 x 30000), and wider
    // rows go to the split plan
    p.block = 1024;
    p.lpr = 1024;
    p.nv = (int)std::max<int64_t>(4, pow2ceil((nvec + 1023) / 1024));
    p.rpi = 1;
  } else {
    // task splitting: S members per row, each a 256-lane workgroup holding
    // <= 16 fragments per lane, or a 1024-lane one holding <= 8.  The softmax
    // family on 16-byte fragments takes 1024-lane members for many rows wider
    // than one of them holds (measured on MI355X, 256- against 1024-lane
    // members: 256 x 65536 34.1 / 29.2 us, 128 x 131072 34.9 / 30.2 us,
    // 2048 x 128256 420.0 / 373.9 us; the norms gain nothing, and few rows or
    // 4-byte fragments lose)
    const bool wide_members = !is_norm(op) && p.w == 4 && 2 * rows >= di->cus && nvec > 1024 * 8;
    const int blk = op != kLayerNormAffine && env_int("CF_SPLIT_BLOCK", wide_members ? 1024 : 256) == 1024 ? 1024 : 256;
    const int64_t per_member = blk == 1024 ? 1024 * 8 : 256 * 16;
    const int64_t s_min = (nvec + per_member - 1) / per_member;
    int64_t S = std::max<int64_t>(s_min, rows >= di->cus ? 1 : pow2ceil((di->cus + rows - 1) / rows));
    if (force_split > 1) S = std::max<int64_t>(force_split, s_min);
    if (S > kMaxSplit) return CF_EUNSUPPORTED;
    const int64_t slice_vec = (nvec + S - 1) / S;
    p.split = (int)S;
    p.block = blk;
    p.nv = blk == 1024 ? (int)std::max<int64_t>(4, pow2ceil((slice_vec + 1023) / 1024)) : pow2ceil((slice_vec + 255) / 256);
    if (p.nv > (blk == 1024 ? 8 : 16)) return CF_EUNSUPPORTED;
    p.slice = slice_vec * p.w;
    p.lpr = blk;
    p.rpi = 1;
  }
  const int rows_per_blk = (p.block / p.lpr) * p.rpi;
  if (p.split == 1) {
    const int64_t nblk = (rows + rows_per_blk - 1) / rows_per_blk;
    const int64_t cap = (int64_t)di->cus * env_int("CF_ROWS_WG_PER_CU", 32);
    p.grid = (int)std::min<int64_t>(nblk, env_int("CF_FORCE_GRID", cap));
  } else {
    int occ = 0;
    if (rows_split_occupancy(op, p, &occ) != hipSuccess || occ <= 0) return CF_EHIP;
    p.occupancy = occ;
    // CF_FORCE_CUS plans for a device with fewer CUs (a test hook for the refusal below)
    const int64_t cap = (int64_t)occ * std::min<long>(di->cus, std::max<long>(1, env_int("CF_FORCE_CUS", di->cus)));
    const int64_t items = rows * p.split;
    int64_t G = std::min<int64_t>(items, cap / p.split * p.split);
    if (G < p.split) return CF_EOCCUPANCY;
    if (G / p.split > kMaxJoins) G = kMaxJoins * p.split;
    p.grid = (int)G;
  }
  *pl = p;
  return CF_OK;
}

// Split plans: per group of S members, 2 parities x 2 fields x S tagged 8-byte
// slots, i.e. 32 bytes per resident workgroup.
size_t rows_ws_bytes(const RowPlan& p, int64_t rows) {
  (void)rows;
  if (p.split <= 1) return 0;
  return ws_layout((int64_t)p.grid * 8).total;
}

void record_rows_plan(const char* name, const RowPlan& p, int64_t rows, int64_t cols) {
  char buf[512];
  snprintf(buf, sizeof buf,
           "{\"call\":\"%s\",\"rows\":%lld,\"cols\":%lld,\"kernel\":\"%s\",\"frag_floats\":%d,"
           "\"lanes_per_row\":%d,\"frags_per_lane\":%d,\"rows_in_flight\":%d,\"split\":%d,"
           "\"slice\":%lld,\"grid\":%d,\"block\":%d,\"aggregation\":\"%s\",\"occupancy\":%d}",
           name, (long long)rows, (long long)cols, p.split > 1 ? "k_rows_split" : "k_rows", p.w, p.lpr,
           p.nv, p.rpi, p.split, (long long)p.slice, p.grid, p.block, p.split > 1 ? "all-read" : "none",
           p.occupancy);
  g_last_plan = buf;
}

cf_status run_rows(const char* name, int op, const float* x, float* y, float* y_pre, const float* v, float pw,
                   float eps, int64_t rows, int64_t cols, void* ws, size_t ws_bytes, hipStream_t st,
                   const float* gamma, const float* beta) {
  if (!x || !y || rows <= 0 || cols <= 0) return CF_EINVAL;
  if (op == kPowSoftmax && !v) return CF_EINVAL;
  if (is_norm(op) && !(eps >= 0.0f)) return CF_EINVAL;
  if (op == kLayerNormAffine && (!gamma || !beta)) return CF_EINVAL;
  const size_t bytes = (size_t)rows * cols * sizeof(float);
  if (overlap(x, bytes, y, bytes)) return CF_EINVAL;
  if (y_pre && (overlap(y_pre, bytes, y, bytes) || overlap(y_pre, bytes, x, bytes))) return CF_EINVAL;
  const size_t vbytes = (size_t)cols * sizeof(float);
  if ((gamma && overlap(y, bytes, gamma, vbytes)) || (beta && overlap(y, bytes, beta, vbytes))) return CF_EINVAL;
  const bool vec_ok = aligned16(x) && aligned16(y) && (!y_pre || aligned16(y_pre)) && (!gamma || aligned16(gamma)) &&
                      (!beta || aligned16(beta));
  RowPlan p;
  cf_status s = plan_rows(op, rows, cols, vec_ok, &p);
  if (s != CF_OK) return s;
  const size_t need = rows_ws_bytes(p, rows);
  if (need > 0 && (!ws || ws_bytes < need)) return CF_EWORKSPACE;
  RowArgs a{};
  a.x = x; a.y = y; a.y_pre = y_pre; a.v = v; a.p = pw; a.eps = eps;
  a.gamma = gamma; a.beta = beta;
  a.rows = rows; a.cols = cols;
  if (need > 0) {
    const WsLayout L = ws_layout((int64_t)p.grid * 8);
    char* base = static_cast<char*>(ws);
    a.err = reinterpret_cast<uint32_t*>(base);
    a.joins = reinterpret_cast<uint64_t*>(base + L.joins_off);
    a.slots = reinterpret_cast<uint64_t*>(base + L.partials_off);
  }
  a.S = p.split;
  a.slice = p.slice;
  record_rows_plan(name, p, rows, cols);
  return launch_rows(op, p, a, st) == hipSuccess ? CF_OK : CF_EHIP;
}

// ------------------------------------------------------------ GEMM planning

// Strip softmax: 128 x 128 tiles; each row block's column tiles are cut into
// S strips of C consecutive tiles (no strip empty), one per resident
// workgroup where the rows allow.
// Strips (softmax, and the softmax between two GEMMs): row-block units of
// contiguous column tiles, 128 x 128 tiles at two workgroups per CU for the
// softmax, 256 rows x 64 keys at one 8-wave workgroup per CU for the
// back-to-back GEMM (its output accumulator needs the registers).
static cf_status plan_gemm_strips(int epi, int64_t M, int64_t N, int64_t K, DevInfo* di, GemmPlan* p0,
                                  GemmPlan* pl) {
  GemmPlan p = *p0;
  p.algo = 2;
  p.nn = 0;
  p.bm = epi == kEpiSoftmaxGemm ? kB2bBM : 128;
  p.bn = epi == kEpiSoftmaxGemm ? kB2bBN : 128;
  p.bk = K <= 32 ? 32 : (K <= 64 ? 64 : 128);  // reduction depth the kernel covers (zero-padded)
  int occ = 0;
  if (gemm_occupancy(epi, p, &occ) != hipSuccess || occ <= 0) return CF_EHIP;
  p.occupancy = occ;
  const int64_t cap = (int64_t)occ * di->cus;
  const int64_t tn = (N + p.bn - 1) / p.bn, tm = (M + p.bm - 1) / p.bm;
  // one join word per row block (the back-to-back GEMM's is its second block of words)
  if ((epi == kEpiSoftmaxGemm ? 2 : 1) * tm > kMaxJoins) return CF_EUNSUPPORTED;
  int64_t S = std::max<int64_t>(1, std::min<int64_t>(tn, cap / tm));
  // the softmax strips hold at least four tiles each: a strip's Q load,
  // publication and join cost about as much as a few tiles.  Measured on
  // MI355X (D = 128, strips: us): 4096 x 4096 16: 31.7, 8: 25.5;
  // 2048 x 8192 32: 40.7, 16: 26.4; 8192 x 2048 8: 27.1-28.2, 4: 24.9;
  // 8192 x 8192 8: 62.3-66.8, 4: 70.1, 16: 67.0
  if (epi == kEpiSoftmax) S = std::max<int64_t>(1, std::min<int64_t>(S, tn / 4));
  const int64_t C = (tn + S - 1) / S;
  S = (tn + C - 1) / C;
  const int64_t units = tm * S;
  p.strips = (int)S;
  p.tiles = (int)(tm * tn);
  p.grid = (int)std::min<int64_t>(units, cap);
  p.rounds = (int)((units + p.grid - 1) / p.grid);
  if (p.rounds > kMaxRounds) return CF_EUNSUPPORTED;
  // the back-to-back GEMM's strips wait for each other's partial outputs:
  // with several strips per row block they must all be resident (one round)
  if (epi == kEpiSoftmaxGemm && S > 1 && p.rounds > 1) return CF_EOCCUPANCY;
  p.leader = true;
  *pl = p;
  return CF_OK;
}

// Workspace of the back-to-back GEMM past the header and join words: the
// strips' partial outputs (strips x M x 128 bf16), then their per-row
// (max, sum) pairs (strips x M float2).
struct B2bLayout {
  size_t opart = 0, total = 0;
};
static B2bLayout b2b_layout(const GemmPlan& p, int64_t M) {
  B2bLayout L;
  L.opart = kPartialsOff;
  L.total = align_up(L.opart + (size_t)M * p.strips * (128 * 2 + 8), 256);
  return L;
}

// the k_gemm_ln2 configuration without pipelining (8 waves, 256 x 256 tiles)
static bool ln_one_at_a_time(int epi, const GemmPlan& p) {
  return epi == kEpiLN && p.algo == 1 && (p.cfg == 0 || p.cfg == 7);
}

cf_status plan_gemm(int epi, bool nn, int64_t M, int64_t N, int64_t K, GemmPlan* pl) {
  DevInfo* di = nullptr;
  cf_status s = dev_info(&di);
  if (s != CF_OK) return s;
  GemmPlan p;
  p.nn = nn ? 1 : 0;
  // softmax with a reduction dimension of at most 128 runs by strips
  const int dalgo = (epi == kEpiSoftmax && K <= 128) ? 2 : 1;
  const bool plain = epi == kEpiStoreF32 || epi == kEpiAct;  // tiles independent of each other
  // activation epilogue: 0 = the round-based kernel (128 x 128 tiles, two
  // workgroups per CU), 1 = large tiles at one 8-wave workgroup per CU, the
  // default where its 256 x 256 tiles fill at least three quarters of the CUs.
  // Measured on MI355X (GELU, K = 1024 unless noted, large against 128 x 128
  // tiles): 4096 x 4096 40.7 / 44.5 us, 8192 x 8192 156.8 / 204.4 us, 4096 x
  // 4096 x 4096 122.1 / 151.5 us; 3072 x 4096 38.8 / 38.5 us; 2048 x 4096 36.3
  // / 24.0 us, 1024 x 4096 33.8 / 18.7 us, 2048 x 2048 x 2048 55.0 / 28.3 us
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  p.algo = epi == kEpiAct ? (int)env_int("CF_GEMM_ACT_ALGO", 4 * big_tiles >= 3 * (int64_t)di->cus ? 1 : 0)
                          : (plain ? 0 : (int)env_int("CF_GEMM_ALGO", dalgo));
  if (epi == kEpiAct && (p.algo < 0 || p.algo > 1)) return CF_EUNSUPPORTED;
  if (p.algo >= 2 && (epi != kEpiSoftmax || K > 128 || p.algo > 2)) return CF_EUNSUPPORTED;
  if (p.algo == 2) return plan_gemm_strips(kEpiSoftmax, M, N, K, di, &p, pl);
  // Default tiles (measured on MI355X): 128x128 at two workgroups per CU for
  // the plain GEMM and the overlapped epilogues, 64x512 for the round-based
  // epilogues.
  // GEMM + LN: the 256 x 256 one-tile-per-workgroup kernel (7) wherever a
  // whole row block of its tiles fits the resident grid and its tiles fill at
  // least half the CUs, else 128 x 128 at two workgroups per CU (3).  Measured
  // on MI355X (K = 1024 unless noted): 64 large tiles, 1024 x 4096 39.9 us
  // against 29.8 us and 2048 x 2048 x 2048 61.1 against 37.5 us; 128 tiles,
  // 2048 x 4096 42.8 against 47.5 us (4096 x 2048: 41.8 against 38.5 us);
  // 256 tiles, 4096 x 4096 49.7 against 63.4 us
  const int dflt = (epi == kEpiAct && p.algo == 1) ? 0
                   : (epi == kEpiLN && p.algo == 1) ? ((N + 255) / 256 <= di->cus && 2 * big_tiles >= di->cus ? 7 : 3)
                                                    : ((plain || p.algo == 1) ? 3 : 4);
  p.cfg = (int)env_int(epi == kEpiSoftmax ? "CF_GEMM_SOFTMAX_CFG"
                       : epi == kEpiLN     ? "CF_GEMM_LN_CFG"
                       : epi == kEpiAct    ? "CF_GEMM_ACT_CFG"
                                           : "CF_GEMM_CFG",
                       dflt);
  if (!gemm_tile_config(epi, p.algo, p.cfg, &p.bm, &p.bn, &p.bk)) return CF_EUNSUPPORTED;
  const int64_t tn = (N + p.bn - 1) / p.bn, tm = (M + p.bm - 1) / p.bm;
  p.tiles = (int)(tn * tm);
  int occ = 0;
  if (gemm_occupancy(epi, p, &occ) != hipSuccess || occ <= 0) return CF_EHIP;
  p.occupancy = occ;
  const int64_t cap = (int64_t)occ * di->cus;
  if (plain) {
    // large-tile activation kernel: persistent, one workgroup per slot
    p.grid = (int)std::min<int64_t>(p.tiles, std::max<int64_t>(cap, 1) * (epi == kEpiAct && p.algo == 1 ? 1 : 4));
  } else if (p.algo == 1) {
    // one join word per row block; every workgroup resident.  Pipelined
    // kernels: a row block's tiles within two consecutive rounds (their
    // progress bound).  The one-tile-at-a-time LN kernel (256 x 256): whole
    // row blocks per round.
    if (tm > kMaxJoins) return CF_EUNSUPPORTED;
    int64_t G = std::min<int64_t>(p.tiles, cap);
    const bool one_at_a_time = ln_one_at_a_time(epi, p);
    if (one_at_a_time) G = std::min<int64_t>(p.tiles, cap / tn * tn);
    if (G < 1 || tn > 2 * G || (one_at_a_time && G < tn)) return CF_EOCCUPANCY;
    if ((p.tiles + G - 1) / G > kMaxRounds) return CF_EUNSUPPORTED;
    p.grid = (int)G;
    // LN: each XCD takes a compact block of every full round's tile grid
    // (sw_a row x sw_b column splits), the one with the fewest A + W bytes
    p.sw_a = p.sw_b = 0;
    if (epi == kEpiLN && env_int("CF_GEMM_SWIZZLE", 0) != 0 && G % 8 == 0 && G % tn == 0) {
      const int64_t rows = G / tn;
      int64_t best = -1;
      for (int sa = 1; sa <= 8; sa *= 2) {
        const int sb = 8 / sa;
        if (rows % sa != 0 || tn % sb != 0) continue;
        const int64_t cost = (rows / sa) * p.bm + (tn / sb) * p.bn;
        if (best < 0 || cost < best) {
          best = cost;
          p.sw_a = sa;
          p.sw_b = sb;
        }
      }
    }
  } else {
    const int64_t G = std::min<int64_t>(p.tiles, cap / tn * tn);
    if (G < tn) return CF_EOCCUPANCY;
    if (G / tn > kMaxJoins) return CF_EUNSUPPORTED;
    p.grid = (int)G;
  }
  p.rounds = (int)((p.tiles + p.grid - 1) / p.grid);
  // [ComFuse] dual-mode inter-CTA aggregation: peer-to-peer for small groups,
  // leader-follower for large ones (threshold from measurement on MI355X).
  const long agg = env_int("CF_AGG_LEADER", -1);
  p.leader = agg >= 0 ? (agg != 0) : (tn > 8);
  *pl = p;
  return CF_OK;
}

// Per-row partials of every column tile (4 floats each, rows rounded up to
// whole row blocks), then 2 floats per row.
size_t gemm_ws_bytes(const GemmPlan& p, int64_t M, int64_t N) {
  const int64_t tn = (N + p.bn - 1) / p.bn, mp = (M + p.bm - 1) / p.bm * p.bm;
  return ws_layout(mp * tn * 4 + M * 2).total;
}

void record_gemm_plan(const char* name, int epi, const GemmPlan& p, int64_t M, int64_t N, int64_t K) {
  const bool plain = epi == kEpiStoreF32 || epi == kEpiAct;
  const bool ov = p.algo >= 1 && !plain;
  const char* kernel = epi == kEpiSoftmaxGemm
                           ? "k_gemm_b2b"
                           : (p.algo == 2 ? "k_gemm_sm3"
                                          : (ov ? (epi == kEpiLN ? (p.cfg == 7 ? "k_gemm_ln3" : "k_gemm_ln2") : "k_gemm_sm2")
                                                : (epi == kEpiAct && p.algo == 1 ? "k_gemm_act2" : "k_gemm")));
  const bool single = ln_one_at_a_time(epi, p);
  const char* sched = epi == kEpiSoftmaxGemm
                          ? "strips, back-to-back"
                          : (p.algo == 2 ? "strips"
                                         : (ov ? (epi == kEpiLN ? (p.cfg == 7   ? "one-tile-per-launch-round"
                                                                  : single      ? "one-tile-at-a-time"
                                                                                : "pipelined")
                                                                : "two-sweep")
                                               : (plain ? "independent-tiles" : "rounds")));
  char buf[512];
  snprintf(buf, sizeof buf,
           "{\"call\":\"%s\",\"M\":%lld,\"N\":%lld,\"K\":%lld,\"kernel\":\"%s\",\"tile\":[%d,%d,%d],"
           "\"layout\":\"%s\",\"tiles\":%d,\"row_group\":%lld,\"grid\":%d,\"block\":%d,\"occupancy\":%d,"
           "\"rounds\":%d,\"aggregation\":\"%s\",\"schedule\":\"%s\",\"xcd_block\":[%d,%d]}",
           name, (long long)M, (long long)N, (long long)K, kernel, p.bm, p.bn, p.bk, p.nn ? "NN" : "NT", p.tiles,
           p.algo == 2 ? (long long)p.strips : (long long)((N + p.bn - 1) / p.bn), p.grid,
           (single || epi == kEpiSoftmaxGemm || (epi == kEpiAct && p.algo == 1)) ? 512 : 256,
           p.occupancy, p.rounds,
           plain ? "none" : ((ov || p.leader) ? (epi == kEpiLN && p.algo == 1 ? "peer-to-peer" : "leader") : "peer-to-peer"),
           sched,
           p.sw_a, p.sw_b);
  g_last_plan = buf;
}

cf_status check_gemm_shape(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return CF_EINVAL;
  if (N % 8 != 0 || K % 8 != 0) return CF_EUNSUPPORTED;
  // every operand is addressed through a buffer descriptor with 32-bit offsets
  // below 2^31 (the out-of-range offset)
  const int64_t lim = (int64_t)1 << 31;
  if (M * K * 2 >= lim || N * K * 2 >= lim || M * N * 2 >= lim) return CF_EUNSUPPORTED;
  // offsets of a tile that overhangs the last row (by at most 256) stay
  // below 2^32, so they land out of range instead of wrapping
  const int64_t lim32 = (int64_t)1 << 32;
  if ((M + 256) * K * 2 >= lim32 || (N + 256) * K * 2 >= lim32 || (M + 256) * N * 2 >= lim32) return CF_EUNSUPPORTED;
  return CF_OK;
}

}  // namespace

// =================================================================== C-ABI

extern "C" {

const char* cf_status_str(cf_status s) {
  switch (s) {
    case CF_OK: return "CF_OK";
    case CF_EINVAL: return "CF_EINVAL: invalid argument";
    case CF_EUNSUPPORTED: return "CF_EUNSUPPORTED: shape not supported";
    case CF_EALIGN: return "CF_EALIGN: pointer not 16-byte aligned";
    case CF_EWORKSPACE: return "CF_EWORKSPACE: workspace missing or too small";
    case CF_EOCCUPANCY: return "CF_EOCCUPANCY: cooperating workgroups cannot all be resident";
    case CF_EHIP: return "CF_EHIP: HIP runtime error";
  }
  return "unknown cf_status";
}

int cf_last_plan(char* buf, size_t n) {
  if (buf && n > 0) {
    const size_t k = std::min(n - 1, g_last_plan.size());
    memcpy(buf, g_last_plan.data(), k);
    buf[k] = 0;
  }
  return (int)g_last_plan.size();
}

cf_status cf_workspace_error(const void* ws, int clear, uint32_t* out, hipStream_t stream) {
  if (!ws || !out) return CF_EINVAL;
  uint32_t w = 0;
  if (hipMemcpyAsync(&w, ws, sizeof w, hipMemcpyDeviceToHost, stream) != hipSuccess) return CF_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return CF_EHIP;
  if (clear) {
    // a fill kernel, not a memset node: the word is one float's bytes
    if (u_fill(static_cast<float*>(const_cast<void*>(ws)), 1, 0.0f, stream) != hipSuccess) return CF_EHIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return CF_EHIP;
  }
  *out = w;
  return CF_OK;
}

size_t cf_workspace_bytes(int op, int64_t d0, int64_t d1, int64_t d2) {
  if (d0 <= 0 || d1 <= 0) return (size_t)-1;
  switch (op) {
    case CF_OP_STITCH_SOFTMAX:
    case CF_OP_STITCH_LAYERNORM:
    case CF_OP_STITCH_POW_BCAST_ADD:
    case CF_OP_STITCH_LAYERNORM_AFFINE:
    case CF_OP_STITCH_RMSNORM: {
      const int rop = op == CF_OP_STITCH_SOFTMAX          ? kSoftmax
                      : op == CF_OP_STITCH_LAYERNORM      ? kLayerNorm
                      : op == CF_OP_STITCH_POW_BCAST_ADD  ? kPowSoftmax
                      : op == CF_OP_STITCH_LAYERNORM_AFFINE ? kLayerNormAffine
                                                            : kRmsNorm;
      RowPlan p;
      if (plan_rows(rop, d0, d1, true, &p) != CF_OK) return (size_t)-1;
      const size_t a = rows_ws_bytes(p, d0);
      RowPlan q;  // the 4-byte-fragment plan may split differently
      if (plan_rows(rop, d0, d1, false, &q) != CF_OK) return (size_t)-1;
      return std::max(a, rows_ws_bytes(q, d0));
    }
    case CF_OP_GEMM_LN:
    case CF_OP_GEMM_SOFTMAX: {
      if (d2 <= 0) return (size_t)-1;
      GemmPlan p;
      if (plan_gemm(op == CF_OP_GEMM_LN ? kEpiLN : kEpiSoftmax, op == CF_OP_GEMM_LN, d0, d1, d2, &p) != CF_OK)
        return (size_t)-1;
      return gemm_ws_bytes(p, d0, d1);
    }
    case CF_OP_GEMM_SOFTMAX_GEMM: {
      if (d2 <= 0 || d2 > 128) return (size_t)-1;
      DevInfo* di = nullptr;
      if (dev_info(&di) != CF_OK) return (size_t)-1;
      GemmPlan p;
      if (plan_gemm_strips(kEpiSoftmaxGemm, d0, d1, d2, di, &p, &p) != CF_OK) return (size_t)-1;
      return b2b_layout(p, d0).total;
    }
    case CF_OP_GEMM_ACT: {
      if (d2 <= 0) return (size_t)-1;
      GemmPlan p;
      if (plan_gemm(kEpiAct, true, d0, d1, d2, &p) != CF_OK) return (size_t)-1;
      return 0;  // the tiles are independent: no partials, no joins
    }
  }
  return (size_t)-1;
}

cf_status cf_stitch_softmax(const float* x, float* y, int64_t rows, int64_t cols, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  return run_rows("cf_stitch_softmax", kSoftmax, x, y, nullptr, nullptr, 0.f, 0.f, rows, cols, ws, ws_bytes, stream,
                  nullptr, nullptr);
}

cf_status cf_stitch_layernorm(const float* x, float* y, int64_t rows, int64_t cols, float eps, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  return run_rows("cf_stitch_layernorm", kLayerNorm, x, y, nullptr, nullptr, 0.f, eps, rows, cols, ws, ws_bytes,
                  stream, nullptr, nullptr);
}

cf_status cf_stitch_pow_bcast_add(const float* x, const float* v, float p, float* y, float* y_pre, int64_t rows,
                                  int64_t cols, void* ws, size_t ws_bytes, hipStream_t stream) {
  return run_rows("cf_stitch_pow_bcast_add", kPowSoftmax, x, y, y_pre, v, p, 0.f, rows, cols, ws, ws_bytes, stream,
                  nullptr, nullptr);
}

cf_status cf_stitch_layernorm_affine(const float* x, const float* gamma, const float* beta, float* y, int64_t rows,
                                     int64_t cols, float eps, void* ws, size_t ws_bytes, hipStream_t stream) {
  return run_rows("cf_stitch_layernorm_affine", kLayerNormAffine, x, y, nullptr, nullptr, 0.f, eps, rows, cols, ws,
                  ws_bytes, stream, gamma, beta);
}

cf_status cf_stitch_rmsnorm(const float* x, const float* gamma, float* y, int64_t rows, int64_t cols, float eps,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  return run_rows("cf_stitch_rmsnorm", kRmsNorm, x, y, nullptr, nullptr, 0.f, eps, rows, cols, ws, ws_bytes, stream,
                  gamma, nullptr);
}

static cf_status run_gemm(const char* name, int epi, bool nn, GemmArgs a, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  GemmPlan p;
  cf_status s = plan_gemm(epi, nn, a.M, a.N, a.K, &p);
  if (s != CF_OK) return s;
  const size_t need = gemm_ws_bytes(p, a.M, a.N);
  if (!ws || ws_bytes < need) return CF_EWORKSPACE;
  const int64_t tn = (a.N + p.bn - 1) / p.bn, tm = (a.M + p.bm - 1) / p.bm;
  const int64_t mp = tm * p.bm;  // rows rounded up to whole row blocks
  const WsLayout L = ws_layout(mp * tn * 4 + a.M * 2);
  char* base = static_cast<char*>(ws);
  a.err = reinterpret_cast<uint32_t*>(base);
  a.joins = reinterpret_cast<uint64_t*>(base + L.joins_off);
  a.partials = reinterpret_cast<float*>(base + L.partials_off);
  a.finals = a.partials + mp * tn * 4;
  a.tiles_n = (int)tn;
  a.tiles_m = (int)tm;
  a.agg_leader = p.leader ? 1 : 0;
  a.strips = p.strips;
  a.sw_a = p.sw_a;
  a.sw_b = p.sw_b;
  record_gemm_plan(name, epi, p, a.M, a.N, a.K);
  return launch_gemm(epi, p, a, stream) == hipSuccess ? CF_OK : CF_EHIP;
}

static cf_status check_gemm_ln_args(const cf_bf16* A, const cf_bf16* W, const float* bias, const cf_bf16* R,
                                    const float* gamma, const float* beta, float eps, cf_bf16* Y, int64_t M,
                                    int64_t N, int64_t K) {
  if (!A || !W || !bias || !gamma || !beta || !Y || !(eps >= 0.0f)) return CF_EINVAL;
  cf_status s = check_gemm_shape(M, N, K);
  if (s != CF_OK) return s;
  if (!aligned16(A) || !aligned16(W) || !aligned16(Y) || !aligned16(bias) || !aligned16(gamma) ||
      !aligned16(beta) || (R && !aligned16(R)))
    return CF_EALIGN;
  const size_t ybytes = (size_t)M * N * 2;
  if (overlap(Y, ybytes, A, (size_t)M * K * 2) || overlap(Y, ybytes, W, (size_t)K * N * 2) ||
      (R && overlap(Y, ybytes, R, ybytes)))
    return CF_EINVAL;
  return CF_OK;
}

cf_status cf_gemm_ln(const cf_bf16* A, const cf_bf16* W, const float* bias, const cf_bf16* R, const float* gamma,
                     const float* beta, float eps, cf_bf16* Y, int64_t M, int64_t N, int64_t K, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  cf_status s = check_gemm_ln_args(A, W, bias, R, gamma, beta, eps, Y, M, N, K);
  if (s != CF_OK) return s;
  GemmArgs a{};
  a.A = A; a.B = W; a.bias = bias; a.R = R; a.gamma = gamma; a.beta = beta; a.eps = eps; a.Y = Y;
  a.M = M; a.N = N; a.K = K;
  return run_gemm("cf_gemm_ln", kEpiLN, true, a, ws, ws_bytes, stream);
}

// ------------------------------------------------ allocation-free GEMM + LN
//
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc): cf_gemm_ln's workspace
// comes from this file-scope device array instead of the caller.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code the
// array's name is only a host-side stand-in, never a device address: the
// device address is looked up once per device, with that device current, and
// only that address is handed to kernels.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct ScratchDev {
  void* ptr = nullptr;
  bool ok = false;
};
ScratchDev g_scratch[kMaxDev];
std::once_flag g_scratch_once[kMaxDev];

static cf_status scratch_on_current_device(void** out) {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= kMaxDev) return CF_EHIP;
  std::call_once(g_scratch_once[d], [d] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess && p != nullptr) {
      g_scratch[d].ptr = p;
      g_scratch[d].ok = true;
    }
  });
  if (!g_scratch[d].ok) return CF_EHIP;
  *out = g_scratch[d].ptr;
  return CF_OK;
}

cf_status cf_gemm_ln_noalloc(const cf_bf16* A, const cf_bf16* W, const float* bias, const cf_bf16* R,
                             const float* gamma, const float* beta, float eps, cf_bf16* Y, int64_t M, int64_t N,
                             int64_t K, hipStream_t stream) {
  cf_status s = check_gemm_ln_args(A, W, bias, R, gamma, beta, eps, Y, M, N, K);
  if (s != CF_OK) return s;
  GemmPlan p;
  s = plan_gemm(kEpiLN, true, M, N, K, &p);
  if (s != CF_OK) return s;
  if (gemm_ws_bytes(p, M, N) > kScratchBytes) return CF_EWORKSPACE;  // the shape needs more than the scratch holds
  void* ws = nullptr;
  s = scratch_on_current_device(&ws);
  if (s != CF_OK) return s;
  // The error word and the join words this plan uses start at zero: cleared by
  // a fill kernel on the caller's stream (no memset node if the stream is
  // being captured), so a call after one whose wait gave up starts clean.
  const int64_t tm = (M + p.bm - 1) / p.bm;
  if (u_fill(static_cast<float*>(ws), (int64_t)(kHeader + tm * sizeof(uint64_t)) / 4, 0.0f, stream) != hipSuccess)
    return CF_EHIP;
  GemmArgs a{};
  a.A = A; a.B = W; a.bias = bias; a.R = R; a.gamma = gamma; a.beta = beta; a.eps = eps; a.Y = Y;
  a.M = M; a.N = N; a.K = K;
  return run_gemm("cf_gemm_ln_noalloc", kEpiLN, true, a, ws, kScratchBytes, stream);
}

cf_status cf_gemm_softmax(const cf_bf16* Q, const cf_bf16* K, float scale, cf_bf16* S, int64_t M, int64_t N,
                          int64_t D, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!Q || !K || !S || !(scale == scale) || scale - scale != 0.0f) return CF_EINVAL;
  cf_status s = check_gemm_shape(M, N, D);
  if (s != CF_OK) return s;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(S)) return CF_EALIGN;
  const size_t sbytes = (size_t)M * N * 2;
  if (overlap(S, sbytes, Q, (size_t)M * D * 2) || overlap(S, sbytes, K, (size_t)N * D * 2)) return CF_EINVAL;
  GemmArgs a{};
  a.A = Q; a.B = K; a.scale = scale; a.Y = S;
  a.M = M; a.N = N; a.K = D;
  return run_gemm("cf_gemm_softmax", kEpiSoftmax, false, a, ws, ws_bytes, stream);
}

static cf_status check_b2b_args(const cf_bf16* Q, const cf_bf16* K, const cf_bf16* V, float scale, cf_bf16* O,
                                int64_t M, int64_t N, int64_t D, int64_t Dv) {
  if (!Q || !K || !V || !O || !(scale == scale) || scale - scale != 0.0f) return CF_EINVAL;
  cf_status s = check_gemm_shape(M, N, D);
  if (s != CF_OK) return s;
  if (Dv <= 0) return CF_EINVAL;
  if (D > 128 || Dv > 128 || Dv % 8 != 0) return CF_EUNSUPPORTED;
  // V and O through 32-bit buffer offsets (with a 128-key block of slack)
  if ((N + 128) * Dv * 2 >= (int64_t)1 << 31 || M * Dv * 2 >= (int64_t)1 << 31) return CF_EUNSUPPORTED;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return CF_EALIGN;
  const size_t ob = (size_t)M * Dv * 2;
  if (overlap(O, ob, Q, (size_t)M * D * 2) || overlap(O, ob, K, (size_t)N * D * 2) ||
      overlap(O, ob, V, (size_t)N * Dv * 2))
    return CF_EINVAL;
  return CF_OK;
}

cf_status cf_gemm_softmax_gemm(const cf_bf16* Q, const cf_bf16* K, const cf_bf16* V, float scale, cf_bf16* O,
                               int64_t M, int64_t N, int64_t D, int64_t Dv, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  cf_status s = check_b2b_args(Q, K, V, scale, O, M, N, D, Dv);
  if (s != CF_OK) return s;
  DevInfo* di = nullptr;
  s = dev_info(&di);
  if (s != CF_OK) return s;
  GemmPlan p;
  s = plan_gemm_strips(kEpiSoftmaxGemm, M, N, D, di, &p, &p);
  if (s != CF_OK) return s;
  const B2bLayout L = b2b_layout(p, M);
  if (!ws || ws_bytes < L.total) return CF_EWORKSPACE;
  if (M * p.strips * 128 * 2 >= (int64_t)1 << 31) return CF_EUNSUPPORTED;  // buffer offsets of the partials
  char* base = static_cast<char*>(ws);
  GemmArgs a{};
  a.A = Q; a.B = K; a.V = V; a.scale = scale; a.Y = O;
  a.M = M; a.N = N; a.K = D; a.Dv = Dv;
  a.err = reinterpret_cast<uint32_t*>(base);
  a.joins = reinterpret_cast<uint64_t*>(base + kHeader);
  a.opart = reinterpret_cast<float*>(base + L.opart);
  a.tiles_n = (int)((N + p.bn - 1) / p.bn);
  a.tiles_m = (int)((M + p.bm - 1) / p.bm);
  a.agg_leader = 1;
  a.strips = p.strips;
  record_gemm_plan("cf_gemm_softmax_gemm", kEpiSoftmaxGemm, p, M, N, D);
  return launch_gemm(kEpiSoftmaxGemm, p, a, stream) == hipSuccess ? CF_OK : CF_EHIP;
}

static cf_status check_act_args(const cf_bf16* A, const cf_bf16* W, const float* bias, int act, cf_bf16* Y,
                                int64_t M, int64_t N, int64_t K) {
  if (!A || !W || !Y || act < CF_ACT_NONE || act > CF_ACT_RSQRT) return CF_EINVAL;
  cf_status s = check_gemm_shape(M, N, K);
  if (s != CF_OK) return s;
  if (!aligned16(A) || !aligned16(W) || !aligned16(Y) || (bias && !aligned16(bias))) return CF_EALIGN;
  const size_t yb = (size_t)M * N * 2;
  if (overlap(Y, yb, A, (size_t)M * K * 2) || overlap(Y, yb, W, (size_t)K * N * 2) ||
      (bias && overlap(Y, yb, bias, (size_t)N * 4)))
    return CF_EINVAL;
  return CF_OK;
}

cf_status cf_gemm_act(const cf_bf16* A, const cf_bf16* W, const float* bias, int act, cf_bf16* Y, int64_t M,
                      int64_t N, int64_t K, void* ws, size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  cf_status s = check_act_args(A, W, bias, act, Y, M, N, K);
  if (s != CF_OK) return s;
  GemmPlan p;
  s = plan_gemm(kEpiAct, true, M, N, K, &p);
  if (s != CF_OK) return s;
  GemmArgs a{};
  a.A = A; a.B = W; a.bias = bias; a.act = act; a.Y = Y;
  a.M = M; a.N = N; a.K = K;
  a.tiles_n = (int)((N + p.bn - 1) / p.bn);
  a.tiles_m = (int)((M + p.bm - 1) / p.bm);
  record_gemm_plan("cf_gemm_act", kEpiAct, p, M, N, K);
  return launch_gemm(kEpiAct, p, a, stream) == hipSuccess ? CF_OK : CF_EHIP;
}

// ------------------------------------------------------------ unfused chains
// Workspace: fp32 intermediates, placed after the header and the join words
// (which they never touch, so one zero-filled workspace serves fused and
// unfused calls alike).  Vectors first (aligned), then full-size buffers.
// Each operator materializes its output.

static char* unfused_base(void* ws) { return static_cast<char*>(ws) + kPartialsOff; }

size_t cf_unfused_workspace_bytes(int op, int64_t d0, int64_t d1, int64_t d2) {
  if (d0 <= 0 || d1 <= 0) return (size_t)-1;
  const size_t vec = align_up((size_t)d0 * 4, 256);
  const size_t full = align_up((size_t)d0 * d1 * 4, 256);
  size_t n = (size_t)-1;
  switch (op) {
    case CF_OP_STITCH_SOFTMAX: n = 2 * vec + 2 * full; break;
    case CF_OP_STITCH_LAYERNORM: n = 4 * vec + 2 * full; break;
    case CF_OP_STITCH_POW_BCAST_ADD: n = 3 * vec + 3 * full; break;
    case CF_OP_STITCH_LAYERNORM_AFFINE: n = 4 * vec + 3 * full; break;
    case CF_OP_STITCH_RMSNORM: n = 3 * vec + 2 * full; break;
    case CF_OP_GEMM_LN: n = d2 > 0 ? 4 * vec + 3 * full : (size_t)-1; break;
    case CF_OP_GEMM_SOFTMAX: n = d2 > 0 ? 2 * vec + 3 * full : (size_t)-1; break;
    case CF_OP_GEMM_ACT: n = d2 > 0 ? 2 * full : (size_t)-1; break;
    case CF_OP_GEMM_SOFTMAX_GEMM:  // + S bf16 [M x N] + the second product fp32 [M x (Dv <= 128)]
      n = d2 > 0 ? 2 * vec + 3 * full + align_up((size_t)d0 * d1 * 2, 256) + align_up((size_t)d0 * 128 * 4, 256)
                 : (size_t)-1;
      break;
  }
  return n == (size_t)-1 ? n : kPartialsOff + n;
}

#define CF_TRY(call)                        \
  do {                                      \
    if ((call) != hipSuccess) return CF_EHIP; \
  } while (0)

static cf_status unfused_softmax_chain(const float* x, float* y, int64_t rows, int64_t cols, char* ws,
                                       hipStream_t st) {
  const size_t vec = align_up((size_t)rows * 4, 256), full = align_up((size_t)rows * cols * 4, 256);
  float* m = reinterpret_cast<float*>(ws);
  float* s = reinterpret_cast<float*>(ws + vec);
  float* d = reinterpret_cast<float*>(ws + 2 * vec);
  float* e = reinterpret_cast<float*>(ws + 2 * vec + full);
  CF_TRY(u_rowreduce(x, m, rows, cols, 1, st));
  CF_TRY(u_bcast_col(x, m, d, rows, cols, 0, st));
  CF_TRY(u_map(d, e, rows * cols, 0, 0.f, 0.f, st));
  CF_TRY(u_rowreduce(e, s, rows, cols, 0, st));
  CF_TRY(u_bcast_col(e, s, y, rows, cols, 1, st));
  return CF_OK;
}

static cf_status unfused_ln_chain(const float* x, float* y, int64_t rows, int64_t cols, float eps, char* ws,
                                  hipStream_t st) {
  const size_t vec = align_up((size_t)rows * 4, 256), full = align_up((size_t)rows * cols * 4, 256);
  float* s = reinterpret_cast<float*>(ws);
  float* mu = reinterpret_cast<float*>(ws + vec);
  float* ss = reinterpret_cast<float*>(ws + 2 * vec);
  float* r = reinterpret_cast<float*>(ws + 3 * vec);
  float* c = reinterpret_cast<float*>(ws + 4 * vec);
  float* q = reinterpret_cast<float*>(ws + 4 * vec + full);
  CF_TRY(u_rowreduce(x, s, rows, cols, 0, st));
  CF_TRY(u_map(s, mu, rows, 4, 1.0f / (float)cols, 0.f, st));
  CF_TRY(u_bcast_col(x, mu, c, rows, cols, 0, st));
  CF_TRY(u_map(c, q, rows * cols, 1, 0.f, 0.f, st));
  CF_TRY(u_rowreduce(q, ss, rows, cols, 0, st));
  CF_TRY(u_map(ss, r, rows, 3, eps, 1.0f / (float)cols, st));
  CF_TRY(u_bcast_col(c, r, y, rows, cols, 2, st));
  return CF_OK;
}

cf_status cf_unfused_stitch_softmax(const float* x, float* y, int64_t rows, int64_t cols, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
  if (!x || !y || rows <= 0 || cols <= 0) return CF_EINVAL;
  if (!ws || ws_bytes < cf_unfused_workspace_bytes(CF_OP_STITCH_SOFTMAX, rows, cols, 0)) return CF_EWORKSPACE;
  g_last_plan = "{\"call\":\"cf_unfused_stitch_softmax\",\"kernels\":5}";
  return unfused_softmax_chain(x, y, rows, cols, unfused_base(ws), stream);
}

cf_status cf_unfused_stitch_layernorm(const float* x, float* y, int64_t rows, int64_t cols, float eps, void* ws,
                                      size_t ws_bytes, hipStream_t stream) {
  if (!x || !y || rows <= 0 || cols <= 0 || !(eps >= 0.f)) return CF_EINVAL;
  if (!ws || ws_bytes < cf_unfused_workspace_bytes(CF_OP_STITCH_LAYERNORM, rows, cols, 0)) return CF_EWORKSPACE;
  g_last_plan = "{\"call\":\"cf_unfused_stitch_layernorm\",\"kernels\":7}";
  return unfused_ln_chain(x, y, rows, cols, eps, unfused_base(ws), stream);
}

cf_status cf_unfused_stitch_pow_bcast_add(const float* x, const float* v, float p, float* y, float* y_pre,
                                          int64_t rows, int64_t cols, void* ws, size_t ws_bytes,
                                          hipStream_t stream) {
  if (!x || !v || !y || rows <= 0 || cols <= 0) return CF_EINVAL;
  if (!ws || ws_bytes < cf_unfused_workspace_bytes(CF_OP_STITCH_POW_BCAST_ADD, rows, cols, 0)) return CF_EWORKSPACE;
  // layout: pv [rows] | softmax chain scratch (2 vectors + 2 full) | Y (full, when y_pre is NULL)
  char* w = unfused_base(ws);
  const size_t vec = align_up((size_t)rows * 4, 256), full = align_up((size_t)rows * cols * 4, 256);
  float* pv = reinterpret_cast<float*>(w);
  char* chain = w + vec;
  float* Y = y_pre ? y_pre : reinterpret_cast<float*>(w + 3 * vec + 2 * full);
  g_last_plan = "{\"call\":\"cf_unfused_stitch_pow_bcast_add\",\"kernels\":7}";
  CF_TRY(u_map(v, pv, rows, 2, p, 0.f, stream));
  CF_TRY(u_bcast_col(x, pv, Y, rows, cols, 3, stream));
  return unfused_softmax_chain(Y, y, rows, cols, chain, stream);
}

cf_status cf_unfused_stitch_layernorm_affine(const float* x, const float* gamma, const float* beta, float* y,
                                             int64_t rows, int64_t cols, float eps, void* ws, size_t ws_bytes,
                                             hipStream_t stream) {
  if (!x || !y || !gamma || !beta || rows <= 0 || cols <= 0 || !(eps >= 0.f)) return CF_EINVAL;
  if (!ws || ws_bytes < cf_unfused_workspace_bytes(CF_OP_STITCH_LAYERNORM_AFFINE, rows, cols, 0)) return CF_EWORKSPACE;
  char* w = unfused_base(ws);
  const size_t vec = align_up((size_t)rows * 4, 256), full = align_up((size_t)rows * cols * 4, 256);
  float* n = reinterpret_cast<float*>(w + 4 * vec + 2 * full);
  {
    const cf_status cs = unfused_ln_chain(x, n, rows, cols, eps, w, stream);  // 7 kernels
    if (cs != CF_OK) return cs;
  }
  float* t = reinterpret_cast<float*>(w + 4 * vec);                     // the chain's first full buffer, free now
  CF_TRY(u_bcast_row(n, gamma, t, rows, cols, 2, stream));              // * gamma
  CF_TRY(u_bcast_row(t, beta, y, rows, cols, 3, stream));               // + beta
  g_last_plan = "{\"call\":\"cf_unfused_stitch_layernorm_affine\",\"kernels\":9}";
  return CF_OK;
}

cf_status cf_unfused_stitch_rmsnorm(const float* x, const float* gamma, float* y, int64_t rows, int64_t cols, float eps,
                                    void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!x || !y || rows <= 0 || cols <= 0 || !(eps >= 0.f)) return CF_EINVAL;
  if (!ws || ws_bytes < cf_unfused_workspace_bytes(CF_OP_STITCH_RMSNORM, rows, cols, 0)) return CF_EWORKSPACE;
  char* w = unfused_base(ws);
  const size_t vec = align_up((size_t)rows * 4, 256), full = align_up((size_t)rows * cols * 4, 256);
  float* ss = reinterpret_cast<float*>(w);
  float* r = reinterpret_cast<float*>(w + vec);
  float* q = reinterpret_cast<float*>(w + 3 * vec);
  float* t = reinterpret_cast<float*>(w + 3 * vec + full);
  CF_TRY(u_map(x, q, rows * cols, 1, 0.f, 0.f, stream));              // square
  CF_TRY(u_rowreduce(q, ss, rows, cols, 0, stream));                  // row sum
  CF_TRY(u_map(ss, r, rows, 3, eps, 1.0f / (float)cols, stream));     // rsqrt(ss / n + eps)
  if (gamma) {
    CF_TRY(u_bcast_col(x, r, t, rows, cols, 2, stream));              // x * r
    CF_TRY(u_bcast_row(t, gamma, y, rows, cols, 2, stream));          // * gamma
  } else {
    CF_TRY(u_bcast_col(x, r, y, rows, cols, 2, stream));
  }
  g_last_plan = "{\"call\":\"cf_unfused_stitch_rmsnorm\",\"kernels\":5}";
  return CF_OK;
}

cf_status cf_unfused_gemm_ln(const cf_bf16* A, const cf_bf16* W, const float* bias, const cf_bf16* R,
                             const float* gamma, const float* beta, float eps, cf_bf16* Y, int64_t M, int64_t N,
                             int64_t K, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!A || !W || !bias || !gamma || !beta || !Y || !(eps >= 0.f)) return CF_EINVAL;
  cf_status s = check_gemm_shape(M, N, K);
  if (s != CF_OK) return s;
  if (!aligned16(A) || !aligned16(W)) return CF_EALIGN;
  if (!ws || ws_bytes < cf_unfused_workspace_bytes(CF_OP_GEMM_LN, M, N, K)) return CF_EWORKSPACE;
  char* w = unfused_base(ws);
  const size_t vec = align_up((size_t)M * 4, 256), full = align_up((size_t)M * N * 4, 256);
  float* z = reinterpret_cast<float*>(w + 4 * vec);
  float* u = reinterpret_cast<float*>(w + 4 * vec + full);
  float* n = reinterpret_cast<float*>(w + 4 * vec + 2 * full);
  GemmPlan p;
  s = plan_gemm(kEpiStoreF32, true, M, N, K, &p);
  if (s != CF_OK) return s;
  GemmArgs a{};
  a.A = A; a.B = W; a.Z = z; a.M = M; a.N = N; a.K = K;
  a.tiles_n = (int)((N + p.bn - 1) / p.bn);
  a.tiles_m = (int)((M + p.bm - 1) / p.bm);
  CF_TRY(launch_gemm(kEpiStoreF32, p, a, stream));
  CF_TRY(u_bcast_row(z, bias, u, M, N, 3, stream));
  if (R) {
    CF_TRY(u_add_bf16(u, R, z, M * N, stream));
  } else {
    CF_TRY(u_copy(u, z, M * N, stream));
  }
  // LN chain on z (uses the 4 vectors and two full buffers u, n)
  float* sv = reinterpret_cast<float*>(w);
  float* mu = reinterpret_cast<float*>(w + vec);
  float* ss = reinterpret_cast<float*>(w + 2 * vec);
  float* r = reinterpret_cast<float*>(w + 3 * vec);
  CF_TRY(u_rowreduce(z, sv, M, N, 0, stream));
  CF_TRY(u_map(sv, mu, M, 4, 1.0f / (float)N, 0.f, stream));
  CF_TRY(u_bcast_col(z, mu, u, M, N, 0, stream));
  CF_TRY(u_map(u, n, M * N, 1, 0.f, 0.f, stream));
  CF_TRY(u_rowreduce(n, ss, M, N, 0, stream));
  CF_TRY(u_map(ss, r, M, 3, eps, 1.0f / (float)N, stream));
  CF_TRY(u_bcast_col(u, r, n, M, N, 2, stream));
  CF_TRY(u_bcast_row(n, gamma, u, M, N, 2, stream));
  CF_TRY(u_bcast_row(u, beta, n, M, N, 3, stream));
  CF_TRY(u_cast_bf16(n, Y, M * N, stream));
  g_last_plan = "{\"call\":\"cf_unfused_gemm_ln\",\"kernels\":13}";
  return CF_OK;
}

cf_status cf_unfused_gemm_softmax(const cf_bf16* Q, const cf_bf16* K, float scale, cf_bf16* S, int64_t M, int64_t N,
                                  int64_t D, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!Q || !K || !S) return CF_EINVAL;
  cf_status s = check_gemm_shape(M, N, D);
  if (s != CF_OK) return s;
  if (!aligned16(Q) || !aligned16(K)) return CF_EALIGN;
  if (!ws || ws_bytes < cf_unfused_workspace_bytes(CF_OP_GEMM_SOFTMAX, M, N, D)) return CF_EWORKSPACE;
  char* w = unfused_base(ws);
  const size_t vec = align_up((size_t)M * 4, 256), full = align_up((size_t)M * N * 4, 256);
  // layout: m [M] | s [M] | B0 | B1 | B2 (full fp32 buffers); each operator
  // reads and writes distinct buffers.
  float* m = reinterpret_cast<float*>(w);
  float* sv = reinterpret_cast<float*>(w + vec);
  float* B0 = reinterpret_cast<float*>(w + 2 * vec);
  float* B1 = reinterpret_cast<float*>(w + 2 * vec + full);
  float* B2 = reinterpret_cast<float*>(w + 2 * vec + 2 * full);
  GemmPlan p;
  s = plan_gemm(kEpiStoreF32, false, M, N, D, &p);
  if (s != CF_OK) return s;
  GemmArgs a{};
  a.A = Q; a.B = K; a.Z = B0; a.M = M; a.N = N; a.K = D;
  a.tiles_n = (int)((N + p.bn - 1) / p.bn);
  a.tiles_m = (int)((M + p.bm - 1) / p.bm);
  CF_TRY(launch_gemm(kEpiStoreF32, p, a, stream));   // P = Q.K^T
  CF_TRY(u_map(B0, B1, M * N, 4, scale, 0.f, stream)); // S1 = scale * P
  CF_TRY(u_rowreduce(B1, m, M, N, 1, stream));        // m = rowmax
  CF_TRY(u_bcast_col(B1, m, B2, M, N, 0, stream));    // d = S1 - m
  CF_TRY(u_map(B2, B0, M * N, 0, 0.f, 0.f, stream));  // e = exp(d)
  CF_TRY(u_rowreduce(B0, sv, M, N, 0, stream));       // s = rowsum
  CF_TRY(u_bcast_col(B0, sv, B1, M, N, 1, stream));   // y = e / s
  CF_TRY(u_cast_bf16(B1, S, M * N, stream));
  g_last_plan = "{\"call\":\"cf_unfused_gemm_softmax\",\"kernels\":8}";
  return CF_OK;
}

cf_status cf_unfused_gemm_softmax_gemm(const cf_bf16* Q, const cf_bf16* K, const cf_bf16* V, float scale,
                                       cf_bf16* O, int64_t M, int64_t N, int64_t D, int64_t Dv, void* ws,
                                       size_t ws_bytes, hipStream_t stream) {
  cf_status s = check_b2b_args(Q, K, V, scale, O, M, N, D, Dv);
  if (s != CF_OK) return s;
  if (!ws || ws_bytes < cf_unfused_workspace_bytes(CF_OP_GEMM_SOFTMAX_GEMM, M, N, D)) return CF_EWORKSPACE;
  const size_t vec = align_up((size_t)M * 4, 256), full = align_up((size_t)M * N * 4, 256);
  char* w = unfused_base(ws);
  cf_bf16* S = reinterpret_cast<cf_bf16*>(w + 2 * vec + 3 * full);
  float* Z = reinterpret_cast<float*>(w + 2 * vec + 3 * full + align_up((size_t)M * N * 2, 256));
  // S = softmax(scale * Q.K^T) through the 8-kernel chain (its own buffers
  // come first in the same workspace), then O = S.V and the cast
  s = cf_unfused_gemm_softmax(Q, K, scale, S, M, N, D, ws, ws_bytes, stream);
  if (s != CF_OK) return s;
  s = check_gemm_shape(M, Dv, N);
  if (s != CF_OK) return s;
  GemmPlan p;
  s = plan_gemm(kEpiStoreF32, true, M, Dv, N, &p);
  if (s != CF_OK) return s;
  GemmArgs a{};
  a.A = S; a.B = V; a.Z = Z; a.M = M; a.N = Dv; a.K = N;
  a.tiles_n = (int)((Dv + p.bn - 1) / p.bn);
  a.tiles_m = (int)((M + p.bm - 1) / p.bm);
  CF_TRY(launch_gemm(kEpiStoreF32, p, a, stream));
  CF_TRY(u_cast_bf16(Z, O, M * Dv, stream));
  g_last_plan = "{\"call\":\"cf_unfused_gemm_softmax_gemm\",\"kernels\":10}";
  return CF_OK;
}

cf_status cf_unfused_gemm_act(const cf_bf16* A, const cf_bf16* W, const float* bias, int act, cf_bf16* Y,
                               int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes, hipStream_t stream) {
  cf_status s = check_act_args(A, W, bias, act, Y, M, N, K);
  if (s != CF_OK) return s;
  if (!ws || ws_bytes < cf_unfused_workspace_bytes(CF_OP_GEMM_ACT, M, N, K)) return CF_EWORKSPACE;
  const size_t full = align_up((size_t)M * N * 4, 256);
  char* w = unfused_base(ws);
  float* B0 = reinterpret_cast<float*>(w);
  float* B1 = reinterpret_cast<float*>(w + full);
  GemmPlan p;
  s = plan_gemm(kEpiStoreF32, true, M, N, K, &p);
  if (s != CF_OK) return s;
  GemmArgs a{};
  a.A = A; a.B = W; a.Z = B0; a.M = M; a.N = N; a.K = K;
  a.tiles_n = (int)((N + p.bn - 1) / p.bn);
  a.tiles_m = (int)((M + p.bm - 1) / p.bm);
  CF_TRY(launch_gemm(kEpiStoreF32, p, a, stream));  // Z = A.W
  int kernels = 2;
  float* cur = B0;
  if (bias) {
    CF_TRY(u_bcast_row(B0, bias, B1, M, N, 3, stream));  // u = Z + bias
    cur = B1;
    ++kernels;
  }
  static const int kMapOp[] = {-1, 5, 6, 7, 1, 8};  // relu, gelu_tanh, silu, square, rsqrt
  if (act != CF_ACT_NONE) {
    float* out = cur == B0 ? B1 : B0;
    CF_TRY(u_map(cur, out, M * N, kMapOp[act], 0.f, 0.f, stream));  // y = act(u)
    cur = out;
    ++kernels;
  }
  CF_TRY(u_cast_bf16(cur, Y, M * N, stream));
  char buf[96];
  snprintf(buf, sizeof buf, "{\"call\":\"cf_unfused_gemm_act\",\"kernels\":%d}", kernels);
  g_last_plan = buf;
  return CF_OK;
}

// ---------------------------------------------------------------- graphs

cf_status cf_graph_begin(hipStream_t stream) {
  return hipStreamBeginCapture(stream, hipStreamCaptureModeGlobal) == hipSuccess ? CF_OK : CF_EHIP;
}

cf_status cf_graph_end(hipStream_t stream, void** exec) {
  if (!exec) return CF_EINVAL;
  hipGraph_t g = nullptr;
  if (hipStreamEndCapture(stream, &g) != hipSuccess || !g) return CF_EHIP;
  hipGraphExec_t e = nullptr;
  const hipError_t r = hipGraphInstantiate(&e, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (r != hipSuccess) return CF_EHIP;
  if (hipGraphUpload(e, stream) != hipSuccess) {
    (void)hipGraphExecDestroy(e);
    return CF_EHIP;
  }
  *exec = e;
  return CF_OK;
}

cf_status cf_graph_launch(void* exec, hipStream_t stream) {
  if (!exec) return CF_EINVAL;
  return hipGraphLaunch(static_cast<hipGraphExec_t>(exec), stream) == hipSuccess ? CF_OK : CF_EHIP;
}

cf_status cf_graph_destroy(void* exec) {
  if (!exec) return CF_EINVAL;
  return hipGraphExecDestroy(static_cast<hipGraphExec_t>(exec)) == hipSuccess ? CF_OK : CF_EHIP;
}

// ---------------------------------------------------------------- utilities

cf_status cf_util_fill_f32(float* p, int64_t n, float value, hipStream_t stream) {
  if (!p || n <= 0 || !aligned16(p)) return CF_EINVAL;
  return u_fill(p, n, value, stream) == hipSuccess ? CF_OK : CF_EHIP;
}

cf_status cf_util_copy_f32(const float* src, float* dst, int64_t n, hipStream_t stream) {
  if (!src || !dst || n <= 0) return CF_EINVAL;
  if (!aligned16(src) || !aligned16(dst)) return CF_EALIGN;
  if (overlap(src, (size_t)n * 4, dst, (size_t)n * 4)) return CF_EINVAL;
  return u_copy(src, dst, n, stream) == hipSuccess ? CF_OK : CF_EHIP;
}

}  // extern "C"
