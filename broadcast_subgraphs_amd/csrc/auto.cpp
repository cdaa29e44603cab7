// Automatic stitching of a memory-intensive graph: schedule, generate one
// HIP kernel, compile it with hiprtc, launch it.
//
// [AStitch] "Making it automatic": dominant ops (reductions, expensive ops
// feeding a broadcast, outputs), index propagation from the dominants
// through one-to-one ops, merging of dominants (preferring the reduction's
// mapping), the passive block-locality check (Regional when producer and
// consumer sit in one workgroup, else Global); "Four stitching schemes"
// (Local / Regional / Global); "Adaptive thread mapping" (lanes per row by
// the row length, several short rows per workgroup).

#include <hip/hip_runtime.h>
#include <hip/hiprtc.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "cf.h"
#include "cf_spec.h"

namespace {

constexpr int kMaxNodes = 256;
constexpr int kMaxSlots = 16;
constexpr int kMaxDevices = 16;
constexpr int kMaxFrags = 8;       // float4 fragments per lane
constexpr int kMaxLanes = 1024;    // lanes per row (one workgroup)
constexpr int kMaxMembers = 256;   // workgroups per row (Global scheme)
// Global-scheme workspace, in the library's fixed layout: the 256-byte header
// (error word at 0), the join-word region (one 64-bit generation-counted word
// per row group), then the tagged partial slots, 8 bytes each.
constexpr int64_t kJoinWords = 16384;
constexpr size_t kSlotsOff = 256 + kJoinWords * 8;

enum Shape { kTile, kRowVal, kVec, kScalar };
enum DomKind { kDomReduce, kDomExpensiveBcast, kDomOutput };
enum Scheme { kLocal, kRegional, kGlobal };

bool is_binary(int op) { return op >= CF_G_ADD && op <= CF_G_POW; }
bool is_unary(int op) { return op >= CF_G_EXP && op <= CF_G_SILU; }
bool is_reduce(int op) { return op == CF_G_ROWSUM || op == CF_G_ROWMAX; }
// ops whose cost is several VALU instructions or a transcendental
bool is_expensive(int op) { return op == CF_G_POW || op == CF_G_DIV || (is_unary(op) && op != CF_G_SQUARE && op != CF_G_RELU); }
const char* op_name(int op) {
  static const char* n[] = {"input", "operand", "matmul", "rowvec", "colvec", "tensor", "const",
                            "add", "sub", "mul", "div", "pow", "exp", "square", "rsqrt", "relu",
                            "gelu_tanh", "silu", "rowsum", "rowmax"};
  return op >= 0 && op <= CF_G_ROWMAX ? n[op] : "-";
}

struct Edge {
  int from, to, scheme;
};

}  // namespace

struct cf_auto {
  int64_t rows = 0, cols = 0;
  std::vector<cf_gnode> g;
  int terminal = -1;
  std::vector<int> shape;
  std::vector<char> live;
  std::vector<std::pair<int, int>> dominants;  // (node, kind)
  std::vector<Edge> edges;
  int lanes = 0, frags = 0, wg = 0, rows_per_wg = 0, waves_per_row = 0;
  bool global = false;  // a row spans `members` workgroups that join at every reduction
  int members = 1, reductions = 0;
  std::string name;  // generated kernel name prefix (unique per graph and mapping)
  std::string src;
  std::vector<char> code;
  std::mutex mu;
  hipModule_t mod[kMaxDevices] = {};
  hipFunction_t fn_vec[kMaxDevices] = {}, fn_scalar[kMaxDevices] = {};
};

namespace {

// ---------------------------------------------------------- scheduling

cf_status infer(cf_auto* A) {
  const int n = (int)A->g.size();
  const cf_gnode* g = A->g.data();
  A->shape.assign(n, -1);
  for (int i = 0; i < n; ++i) {
    const int op = g[i].op;
    auto in_ok = [&](int j) { return j >= 0 && j < i; };
    switch (op) {
      case CF_G_INPUT:
      case CF_G_ROWVEC:
      case CF_G_COLVEC:
      case CF_G_CONST:
        if (g[i].in0 != -1 || g[i].in1 != -1) return CF_EINVAL;
        if (op != CF_G_CONST && (g[i].slot < 0 || g[i].slot >= kMaxSlots)) return CF_EINVAL;
        if (op == CF_G_CONST && !std::isfinite(g[i].value)) return CF_EINVAL;
        A->shape[i] = op == CF_G_INPUT ? kTile : op == CF_G_ROWVEC ? kVec : op == CF_G_COLVEC ? kRowVal : kScalar;
        continue;
      case CF_G_OPERAND:
      case CF_G_MATMUL:
      case CF_G_TENSOR:
        return CF_EUNSUPPORTED;  // compute-intensive roots and bf16 tensors take the GEMM entry points
      default:
        break;
    }
    if (op < CF_G_ADD || op > CF_G_ROWMAX) return CF_EINVAL;
    const int ni = is_binary(op) ? 2 : 1;
    if (!in_ok(g[i].in0) || (ni == 2 ? !in_ok(g[i].in1) : g[i].in1 != -1)) return CF_EINVAL;
    const int sa = A->shape[g[i].in0];
    if (is_reduce(op)) {
      if (sa != kTile) return CF_EUNSUPPORTED;
      A->shape[i] = kRowVal;
    } else if (is_unary(op)) {
      if (sa == kVec) return CF_EUNSUPPORTED;
      A->shape[i] = sa == kScalar ? kScalar : sa;
    } else {
      const int sb = A->shape[g[i].in1];
      if (op == CF_G_POW && sb != kScalar) return CF_EUNSUPPORTED;
      if ((sa == kVec && sb != kTile) || (sb == kVec && sa != kTile)) return CF_EUNSUPPORTED;
      A->shape[i] = (sa == kTile || sb == kTile) ? kTile : (sa == kRowVal || sb == kRowVal) ? kRowVal : kScalar;
    }
  }
  return CF_OK;
}

void mark_live(const cf_gnode* g, int t, std::vector<char>& live) {
  if (t < 0 || live[t]) return;
  live[t] = 1;
  mark_live(g, g[t].in0, live);
  if (is_binary(g[t].op)) mark_live(g, g[t].in1, live);
}

cf_status schedule(cf_auto* A) {
  const int n = (int)A->g.size();
  const cf_gnode* g = A->g.data();
  A->live.assign(n, 0);
  mark_live(g, A->terminal, A->live);
  if (A->shape[A->terminal] != kTile) return CF_EUNSUPPORTED;
  bool has_input = false;
  for (int i = 0; i < n; ++i) has_input |= A->live[i] && g[i].op == CF_G_INPUT;
  if (!has_input) return CF_EUNSUPPORTED;
  // Dominants: every reduction; every expensive op whose per-row result is
  // read by a tile op (computed once per row, then broadcast); the output.
  for (int i = 0; i < n; ++i) {
    if (!A->live[i]) continue;
    if (is_reduce(g[i].op)) A->dominants.push_back({i, kDomReduce});
    if (A->shape[i] == kRowVal && is_expensive(g[i].op)) {
      bool feeds_tile = false;
      for (int j = i + 1; j < n; ++j)
        if (A->live[j] && A->shape[j] == kTile && (g[j].in0 == i || (is_binary(g[j].op) && g[j].in1 == i)))
          feeds_tile = true;
      if (feeds_tile) A->dominants.push_back({i, kDomExpensiveBcast});
    }
  }
  A->dominants.push_back({A->terminal, kDomOutput});
  // Adaptive thread mapping: lanes per row by the row length (at most 4
  // fragments per lane while the row has room, at least 8 lanes, at most one
  // workgroup); short rows pack several to a 256-lane workgroup.
  const int64_t c4 = (A->cols + 3) / 4;
  int lanes = 8;
  while (lanes < kMaxLanes && (int64_t)lanes * 4 < c4) lanes *= 2;
  int64_t frags = (c4 + lanes - 1) / lanes;
  for (int i = 0; i < n; ++i) A->reductions += A->live[i] && is_reduce(g[i].op);
  if (frags > kMaxFrags) {
    // Global: the row is cut into slices of 256 lanes x 8 fragments, one
    // workgroup each; the members of a row publish every reduction's partial,
    // join and merge the partials in member order.
    lanes = 256;
    frags = kMaxFrags;
    const int64_t members = (c4 + (int64_t)lanes * frags - 1) / ((int64_t)lanes * frags);
    if (members > kMaxMembers) return CF_EUNSUPPORTED;
    A->global = true;
    A->members = (int)members;
  }
  A->lanes = lanes;
  A->frags = (int)frags;
  A->wg = std::max(256, lanes);
  A->rows_per_wg = A->wg / lanes;
  A->waves_per_row = std::max(1, lanes / 64);
  // Index propagation and the locality check, per edge: one-to-one edges and
  // per-row values stay in the thread (Local); a reduction's result crosses
  // waves through LDS when a row spans several waves of the workgroup
  // (Regional), else lane shuffles within the wave keep it Local.  All
  // dominants share the row mapping, so they merge into one group.
  for (int j = 0; j < n; ++j) {
    if (!A->live[j] || g[j].op == CF_G_INPUT || g[j].op == CF_G_ROWVEC || g[j].op == CF_G_COLVEC ||
        g[j].op == CF_G_CONST)
      continue;
    const int ni = is_binary(g[j].op) ? 2 : 1;
    for (int q = 0; q < ni; ++q) {
      const int i = q == 0 ? g[j].in0 : g[j].in1;
      const int scheme = !is_reduce(g[i].op) ? kLocal : A->global ? kGlobal : A->waves_per_row > 1 ? kRegional : kLocal;
      A->edges.push_back({i, j, scheme});
    }
  }
  return CF_OK;
}

// ---------------------------------------------------------- code generation

std::string flt(double v) {
  char b[48];
  snprintf(b, sizeof b, "%.9gf", v);
  std::string s = b;
  if (s.find_first_of(".e") == std::string::npos) s.insert(s.size() - 1, ".0");
  if (s == "inff") return "__builtin_inff()";
  return s;
}

// Expression of node i for element (f, e) (tiles and row vectors) or the
// row (per-row values and constants).
std::string ref(const cf_auto* A, int i) {
  const int sh = A->shape[i];
  if (sh == kTile || sh == kVec) return "t" + std::to_string(i) + "[f][e]";
  return "r" + std::to_string(i);
}

std::string apply(int op, const std::string& a, const std::string& b) {
  switch (op) {
    case CF_G_ADD: return "(" + a + " + " + b + ")";
    case CF_G_SUB: return "(" + a + " - " + b + ")";
    case CF_G_MUL: return "(" + a + " * " + b + ")";
    case CF_G_DIV: return "(" + a + " * __builtin_amdgcn_rcpf(" + b + "))";
    case CF_G_POW: return "cf_pow(" + a + ", " + b + ")";
    case CF_G_EXP: return "__builtin_amdgcn_exp2f(1.44269504088896341f * " + a + ")";
    case CF_G_SQUARE: return "(" + a + " * " + a + ")";
    case CF_G_RSQRT: return "__builtin_amdgcn_rsqf(" + a + ")";
    case CF_G_RELU: return "fmaxf(" + a + ", 0.0f)";
    // u * sigmoid(2z), z = sqrt(2/pi)(u + 0.044715 u^3): the tanh form of GELU
    case CF_G_GELU_TANH:
      return "(" + a + " * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(" + a + " * fmaf(-0.1029432395800235f, " +
             a + " * " + a + ", -2.302208198144325f))))";
    case CF_G_SILU: return "(" + a + " * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504088896341f * " + a + ")))";
  }
  return "0.0f";
}

std::string body(const cf_auto* A, bool vec) {
  const int n = (int)A->g.size();
  const cf_gnode* g = A->g.data();
  const int F = A->frags;
  std::string s;
  char b[4096];
  int kr = 0;  // reduction index within the row (Global partial buffers)
  auto loop = [&](const std::string& stmt) {
    s += "#pragma unroll\n      for (int f = 0; f < " + std::to_string(F) +
         "; ++f)\n#pragma unroll\n        for (int e = 0; e < 4; ++e) " + stmt + "\n";
  };
  for (int i = 0; i < n; ++i) {
    if (!A->live[i]) continue;
    const int op = g[i].op, sh = A->shape[i];
    const std::string ti = "t" + std::to_string(i), ri = "r" + std::to_string(i);
    if (op == CF_G_INPUT || op == CF_G_ROWVEC) {
      const bool row = op == CF_G_INPUT;
      const std::string base = std::string("a.p[") + std::to_string(g[i].slot) + "]" + (row ? " + row * cols" : "");
      s += "      float " + ti + "[" + std::to_string(F) + "][4];\n";
      if (vec) {
        snprintf(b, sizeof b,
                 "#pragma unroll\n      for (int f = 0; f < %d; ++f) {\n"
                 "        const long c = c0 + 4L * (f * %d + rl);\n"
                 "        f4 q = {0.f, 0.f, 0.f, 0.f};\n"
                 "        if (%sc < cols) q = %s((const f4*)(%s + c));\n"
                 "        %s[f][0] = q.x; %s[f][1] = q.y; %s[f][2] = q.z; %s[f][3] = q.w;\n      }\n",
                 F, A->lanes, row ? "rok && " : "", row ? "ntld4" : "*", base.c_str(), ti.c_str(), ti.c_str(),
                 ti.c_str(), ti.c_str());
      } else {
        snprintf(b, sizeof b,
                 "#pragma unroll\n      for (int f = 0; f < %d; ++f)\n#pragma unroll\n        for (int e = 0; e < 4; ++e) {\n"
                 "          const long c = c0 + 4L * (f * %d + rl) + e;\n"
                 "          %s[f][e] = (%sc < cols) ? (%s)[c] : 0.0f;\n        }\n",
                 F, A->lanes, ti.c_str(), row ? "rok && " : "", base.c_str());
      }
      s += b;
      continue;
    }
    if (op == CF_G_COLVEC) {
      s += "      const float " + ri + " = rok ? a.p[" + std::to_string(g[i].slot) + "][row] : 0.0f;\n";
      continue;
    }
    if (op == CF_G_CONST) {
      s += "      const float " + ri + " = " + flt(g[i].value) + ";\n";
      continue;
    }
    if (is_reduce(op)) {
      const bool mx = op == CF_G_ROWMAX;
      const std::string init = mx ? "-__builtin_inff()" : "0.0f";
      const std::string comb = mx ? "fmaxf" : "cf_add";
      if (A->global && kr == 0) {
        // Global, a launch's first row: the launch join the kernel arrived on
        // before its first loads completes here, so no member reads a slot
        // before every member has cleared its own
        s += "      if (it_ == 0) {\n"
             "        if (threadIdx.x == 0) cf_await(a.joins + rs, jold, (unsigned)S, a.err);\n"
             "        __syncthreads();\n"
             "      }\n";
      }
      s += "      float " + ri + " = " + init + ";\n";
      snprintf(b, sizeof b, "{ if (c0 + 4L * (f * %d + rl) + e < cols) %s = %s(%s, t%d[f][e]); }", A->lanes, ri.c_str(),
               comb.c_str(), ri.c_str(), g[i].in0);
      loop(b);
      for (int m = std::min(A->lanes, 64) / 2; m >= 1; m /= 2) {
        snprintf(b, sizeof b, "      %s = %s(%s, __shfl_xor(%s, %d, 64));\n", ri.c_str(), comb.c_str(), ri.c_str(),
                 ri.c_str(), m);
        s += b;
      }
      if (A->waves_per_row > 1) {
        // Regional: the row's waves combine through LDS (two alternating slots,
        // one barrier per reduction), in wave order on every lane.  A workgroup
        // may hold several rows (128 lanes per row: two rows of two waves), so
        // each row reads the entries of its own waves, from its first wave on
        snprintf(b, sizeof b,
                 "      if ((threadIdx.x & 63) == 0) red[slot][threadIdx.x >> 6] = %s;\n"
                 "      __syncthreads();\n"
                 "      %s = red[slot][(threadIdx.x >> 6) & ~%du];\n"
                 "#pragma unroll\n      for (int w = 1; w < %d; ++w) %s = %s(%s, red[slot][((threadIdx.x >> 6) & ~%du) + w]);\n"
                 "      slot ^= 1;\n",
                 ri.c_str(), ri.c_str(), A->waves_per_row - 1, A->waves_per_row, ri.c_str(), comb.c_str(),
                 ri.c_str(), A->waves_per_row - 1);
        s += b;
      }
      if (A->global) {
        // Global: publish this member's partial in its tagged slot, take every
        // member's slot once it carries this row's tag (the value arrives with
        // the tag: no separate arrival or load), then a fixed-order merge by
        // the first wave (the same order, so the same bits, on every member)
        snprintf(b, sizeof b,
                 "      {\n"
                 "        unsigned long long* const pp = a.slots + ((rs * 2L + par) * %d + %d) * (long)S;\n"
                 "        const unsigned tag = it_ + 1u;\n"
                 "        if (threadIdx.x == 0) cf_put(pp + sl, tag, %s);\n"
                 "        for (int q = threadIdx.x; q < S; q += (int)blockDim.x) pm[q] = cf_take(pp + q, tag, a.err);\n"
                 "        __syncthreads();\n"
                 "        if (threadIdx.x < 64) {\n"
                 "          float v = %s;\n"
                 "          for (int q = threadIdx.x; q < S; q += 64) v = %s(v, pm[q]);\n"
                 "          for (int m = 32; m >= 1; m >>= 1) v = %s(v, __shfl_xor(v, m, 64));\n"
                 "          if (threadIdx.x == 0) pm[256] = v;\n"
                 "        }\n"
                 "        __syncthreads();\n"
                 "        %s = pm[256];\n"
                 "        __syncthreads();\n"
                 "      }\n",
                 A->reductions, kr, ri.c_str(), init.c_str(), comb.c_str(), comb.c_str(), ri.c_str());
        s += b;
        ++kr;
      }
      continue;
    }
    const int a0 = g[i].in0, a1 = is_binary(op) ? g[i].in1 : -1;
    if (sh == kTile) {
      s += "      float " + ti + "[" + std::to_string(F) + "][4];\n";
      std::string x = ref(A, a0), y = a1 >= 0 ? ref(A, a1) : "";
      if (op == CF_G_DIV && a1 >= 0 && A->shape[a1] != kTile && A->shape[a1] != kVec) {
        // one reciprocal per row, then a product per element
        s += "      const float rc" + std::to_string(i) + " = __builtin_amdgcn_rcpf(" + y + ");\n";
        loop(ti + "[f][e] = " + x + " * rc" + std::to_string(i) + ";");
      } else {
        loop(ti + "[f][e] = " + apply(op, x, y) + ";");
      }
    } else {
      s += "      const float " + ri + " = " + apply(op, ref(A, a0), a1 >= 0 ? ref(A, a1) : "") + ";\n";
    }
  }
  // output
  const std::string to = "t" + std::to_string(A->terminal);
  if (vec) {
    snprintf(b, sizeof b,
             "#pragma unroll\n      for (int f = 0; f < %d; ++f) {\n"
             "        const long c = c0 + 4L * (f * %d + rl);\n"
             "        if (rok && c < cols) {\n"
             "          const f4 q = {%s[f][0], %s[f][1], %s[f][2], %s[f][3]};\n"
             "          __builtin_nontemporal_store(q, (f4*)(a.out + row * cols + c));\n        }\n      }\n",
             F, A->lanes, to.c_str(), to.c_str(), to.c_str(), to.c_str());
  } else {
    snprintf(b, sizeof b,
             "#pragma unroll\n      for (int f = 0; f < %d; ++f)\n#pragma unroll\n        for (int e = 0; e < 4; ++e) {\n"
             "          const long c = c0 + 4L * (f * %d + rl) + e;\n"
             "          if (rok && c < cols) a.out[row * cols + c] = %s[f][e];\n        }\n",
             F, A->lanes, to.c_str());
  }
  s += b;
  return s;
}

std::string generate(const cf_auto* A) {
  std::string s;
  char b[4096];
  s += "// generated: one stitched kernel for a memory-intensive graph\n"
       "typedef float f4 __attribute__((ext_vector_type(4)));\n"
       "struct AutoArgs { const float* p[16]; float* out; long rows; long cols; unsigned* err;\n"
       "                  unsigned long long* joins; unsigned long long* slots; int S; int RG; };\n"
       "// a tagged slot {tag:32 | value:32}: one 64-bit device-scope store publishes\n"
       "// the value together with its tag, so a reader needs no other ordering\n"
       "__device__ __forceinline__ void cf_put(unsigned long long* s, unsigned tag, float v) {\n"
       "  __hip_atomic_store(s, ((unsigned long long)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,\n"
       "                     __HIP_MEMORY_SCOPE_AGENT);\n}\n"
       "// the slot's value once it carries `tag` (capped spin: on giving up, the\n"
       "// error word is set and 0 returned, so the kernel still finishes)\n"
       "__device__ __forceinline__ float cf_take(unsigned long long* s, unsigned tag, unsigned* err) {\n"
       "  for (unsigned it = 0; it < (1u << 20); ++it) {\n"
       "    const unsigned long long w = __hip_atomic_load(s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);\n"
       "    if ((unsigned)(w >> 32) == tag) return __uint_as_float((unsigned)w);\n"
       "    __builtin_amdgcn_s_sleep(1);\n  }\n"
       "  __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);\n"
       "  return 0.0f;\n}\n"
       "// a generation-counted join word {generation:32 | arrivals:32}: arrive (the\n"
       "// returned word is the arrival's), then await: the last of `m` members\n"
       "// advances the generation, the others wait for it (capped spin)\n"
       "__device__ __forceinline__ unsigned long long cf_arrive(unsigned long long* j) {\n"
       "  return __hip_atomic_fetch_add(j, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);\n}\n"
       "__device__ __forceinline__ void cf_await(unsigned long long* j, unsigned long long old, unsigned m,\n"
       "                                         unsigned* err) {\n"
       "  const unsigned gen0 = (unsigned)(old >> 32);\n"
       "  if ((unsigned)old == m - 1) {\n"
       "    __hip_atomic_fetch_add(j, (1ull << 32) - m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);\n"
       "    return;\n  }\n"
       "  for (unsigned it = 0; it < (1u << 20); ++it) {\n"
       "    const unsigned long long w = __hip_atomic_load(j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);\n"
       "    if ((unsigned)(w >> 32) != gen0) return;\n"
       "    __builtin_amdgcn_s_sleep(1);\n  }\n"
       "  __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);\n}\n"
       "__device__ __forceinline__ float cf_add(float x, float y) { return x + y; }\n"
       "// a^b as the real power: an integral exponent is real for either sign of\n"
       "// a (square and multiply up to |b| = 16, else 2^(b log2|a|) with the sign\n"
       "// of an odd power) and a^0 = 1, 0^0 included; any other exponent is\n"
       "// 2^(b log2 a), which is NaN for a negative base, as the real power is\n"
       "__device__ __forceinline__ float cf_pow(float a, float b) {\n"
       "  if (b == __builtin_rintf(b)) {\n"
       "    const float n = __builtin_fabsf(b);\n"
       "    float r;\n"
       "    if (n <= 16.0f) {\n"
       "      r = 1.0f;\n"
       "      float q = a;\n"
       "      for (int k = (int)n; k != 0; k >>= 1) {\n"
       "        if (k & 1) r *= q;\n"
       "        q *= q;\n"
       "      }\n"
       "    } else {\n"
       "      r = __builtin_amdgcn_exp2f(n * __builtin_amdgcn_logf(__builtin_fabsf(a)));\n"
       "      if (a < 0.0f && n * 0.5f != __builtin_truncf(n * 0.5f)) r = -r;\n"
       "    }\n"
       "    return b < 0.0f ? 1.0f / r : r;\n"
       "  }\n"
       "  return __builtin_amdgcn_exp2f(b * __builtin_amdgcn_logf(a));\n"
       "}\n"
       "__device__ __forceinline__ f4 ntld4(const f4* p) { return __builtin_nontemporal_load(p); }\n";
  for (int vec = 1; vec >= 0; --vec) {
    if (A->global) {
      // one row per group of S member workgroups; rows in rounds of RG groups
      snprintf(b, sizeof b,
               "extern \"C\" __global__ __launch_bounds__(%d) void %s_%s(AutoArgs a) {\n"
               "  const long rows = a.rows, cols = a.cols;\n"
               "  const int rl = threadIdx.x;\n"
               "  __shared__ float red[2][16]; int slot = 0;\n"
               "  __shared__ float pm[257];  // the members' partials, then their merge\n"
               "  const int S = a.S, sl = (int)blockIdx.x %% S;\n"
               "  const long rs = (long)blockIdx.x / S;\n"
               "  const long c0 = 4L * sl * %d;\n"
               "  unsigned it_ = 0;  // this launch's rows of the group so far (tags count from 1)\n",
               A->wg, A->name.c_str(), vec ? "vec" : "scalar", A->lanes * A->frags);
      s += b;
      if (A->reductions > 0) {
        snprintf(b, sizeof b,
                 "  // the launch join, before any load: this member clears its slots (both\n"
                 "  // parities, every reduction) and arrives; it awaits the others at its\n"
                 "  // first reduction, so the join overlaps the first row's loads.  No slot\n"
                 "  // read in this launch then holds a value from before it (this kernel's\n"
                 "  // or another op's sharing the workspace), and tags restart at 1\n"
                 "  unsigned long long jold = 0;\n"
                 "  if (threadIdx.x == 0) {\n"
                 "    for (int p = 0; p < 2; ++p)\n"
                 "      for (int k = 0; k < %d; ++k)\n"
                 "        __hip_atomic_store(a.slots + ((rs * 2L + p) * %d + k) * (long)S + sl, 0ull, __ATOMIC_RELAXED,\n"
                 "                           __HIP_MEMORY_SCOPE_AGENT);\n"
                 "    __builtin_amdgcn_s_waitcnt(0);\n"
                 "    jold = cf_arrive(a.joins + rs);\n"
                 "  }\n",
                 A->reductions, A->reductions);
        s += b;
      }
      snprintf(b, sizeof b,
               "  int par = 0;\n"
               "  for (long row = rs; row < rows; row += a.RG, par ^= 1, ++it_) {\n"
               "    const bool rok = true;\n"
               "    {\n");
    } else {
      snprintf(b, sizeof b,
               "extern \"C\" __global__ __launch_bounds__(%d) void %s_%s(AutoArgs a) {\n"
               "  const long rows = a.rows, cols = a.cols;\n"
               "  const int rl = threadIdx.x %% %d, rg = threadIdx.x / %d;\n"
               "  const long c0 = 0;\n"
               "  %s\n"
               "  for (long rb = (long)blockIdx.x * %d; rb < rows; rb += (long)gridDim.x * %d) {\n"
               "    const long row = rb + rg;\n"
               "    const bool rok = row < rows;\n"
               "    {\n",
               A->wg, A->name.c_str(), vec ? "vec" : "scalar", A->lanes, A->lanes,
               A->waves_per_row > 1 ? "__shared__ float red[2][16]; int slot = 0;" : "", A->rows_per_wg,
               A->rows_per_wg);
    }
    s += b;
    s += body(A, vec != 0);
    s += "    }\n  }\n";
    s += "}\n";
  }
  return s;
}

cf_status compile(cf_auto* A) {
  hiprtcProgram p;
  if (hiprtcCreateProgram(&p, A->src.c_str(), "cf_auto.hip", 0, nullptr, nullptr) != HIPRTC_SUCCESS) return CF_EHIP;
  const char* opts[] = {"--offload-arch=gfx950", "-O3", "-ffp-contract=fast",
                        // packed-FP32 VALU forms stay disabled, as for the library's own kernels
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"};
  const hiprtcResult r = hiprtcCompileProgram(p, (int)(sizeof(opts) / sizeof(opts[0])), opts);
  cf_status st = CF_OK;
  if (r != HIPRTC_SUCCESS) {
    size_t ls = 0;
    hiprtcGetProgramLogSize(p, &ls);
    std::string log(ls + 1, '\0');
    hiprtcGetProgramLog(p, &log[0]);
    fprintf(stderr, "cf_auto_build: hiprtc failed:\n%s\n", log.c_str());
    st = CF_EHIP;
  } else {
    size_t cs = 0;
    hiprtcGetCodeSize(p, &cs);
    A->code.resize(cs);
    hiprtcGetCode(p, A->code.data());
  }
  hiprtcDestroyProgram(&p);
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

}  // namespace

extern "C" {

cf_status cf_auto_build(const cf_gnode* nodes, int n, int terminal, int64_t rows, int64_t cols, cf_auto** out) {
  if (!out) return CF_EINVAL;
  *out = nullptr;
  if (!nodes || n <= 0 || n > kMaxNodes || terminal < 0 || terminal >= n || rows <= 0 || cols <= 0) return CF_EINVAL;
  if (rows * cols >= ((int64_t)1 << 40)) return CF_EUNSUPPORTED;
  cf_auto* A = new cf_auto;
  A->rows = rows;
  A->cols = cols;
  A->g.assign(nodes, nodes + n);
  A->terminal = terminal;
  cf_status st = infer(A);
  if (st == CF_OK) st = schedule(A);
  if (st == CF_OK) {
    // name: FNV-1a of the live graph and the mapping, so profiles tell generated kernels apart
    uint64_t h = 1469598103934665603ull;
    auto mix = [&](const void* p, size_t n) {
      for (size_t i = 0; i < n; ++i) h = (h ^ static_cast<const unsigned char*>(p)[i]) * 1099511628211ull;
    };
    for (size_t i = 0; i < A->g.size(); ++i)
      if (A->live[i]) {
        const cf_gnode& q = A->g[i];
        const int32_t f[5] = {q.op, q.in0, q.in1, q.attr, q.slot};
        mix(f, sizeof f);
        mix(&q.value, sizeof q.value);
      }
    const int m[2] = {A->lanes, A->frags};
    mix(m, sizeof m);
    char nm[32];
    snprintf(nm, sizeof nm, "k_auto_%08x", (unsigned)(h ^ (h >> 32)));
    A->name = nm;
    A->src = generate(A);
    st = compile(A);
  }
  if (st != CF_OK) {
    delete A;
    return st;
  }
  *out = A;
  return CF_OK;
}

int cf_auto_describe(const cf_auto* A, char* buf, size_t n) {
  if (!A) return -1;
  static const char* dk[] = {"reduce", "expensive_broadcast", "output"};
  static const char* sk[] = {"local", "regional", "global"};
  char t[512];
  snprintf(t, sizeof t,
           "{\"rows\":%lld,\"cols\":%lld,\"mapping\":{\"lanes_per_row\":%d,\"frags_per_lane\":%d,\"workgroup\":%d,"
           "\"rows_per_workgroup\":%d,\"waves_per_row\":%d,\"workgroups_per_row\":%d},\"dominants\":[",
           (long long)A->rows, (long long)A->cols, A->lanes, A->frags, A->wg, A->rows_per_wg, A->waves_per_row,
           A->members);
  std::string j = t;
  for (size_t d = 0; d < A->dominants.size(); ++d) {
    snprintf(t, sizeof t, "%s{\"node\":%d,\"op\":\"%s\",\"kind\":\"%s\"}", d ? "," : "", A->dominants[d].first,
             op_name(A->g[A->dominants[d].first].op), dk[A->dominants[d].second]);
    j += t;
  }
  j += "],\"groups\":[{\"id\":0,\"mapping\":\"row\",\"dominants\":[";
  for (size_t d = 0; d < A->dominants.size(); ++d) j += (d ? "," : "") + std::to_string(A->dominants[d].first);
  j += "]}],\"edges\":[";
  for (size_t e = 0; e < A->edges.size(); ++e) {
    snprintf(t, sizeof t, "%s{\"from\":%d,\"to\":%d,\"scheme\":\"%s\"}", e ? "," : "", A->edges[e].from,
             A->edges[e].to, sk[A->edges[e].scheme]);
    j += t;
  }
  j += "],\"params\":[";
  bool first = true;
  for (size_t i = 0; i < A->g.size(); ++i) {
    const int op = A->g[i].op;
    if (!A->live[i] || (op != CF_G_INPUT && op != CF_G_ROWVEC && op != CF_G_COLVEC)) continue;
    snprintf(t, sizeof t, "%s{\"slot\":%d,\"kind\":\"%s\",\"node\":%zu}", first ? "" : ",", A->g[i].slot, op_name(op), i);
    j += t;
    first = false;
  }
  snprintf(t, sizeof t, "],\"kernels\":1,\"kernel\":\"%s_vec\",\"source_bytes\":%zu,\"code_bytes\":%zu}",
           A->name.c_str(), A->src.size(), A->code.size());
  j += t;
  if (buf && n > 0) {
    const size_t m = std::min(n - 1, j.size());
    memcpy(buf, j.data(), m);
    buf[m] = 0;
  }
  return (int)j.size();
}

int cf_auto_source(const cf_auto* A, char* buf, size_t n) {
  if (!A) return -1;
  if (buf && n > 0) {
    const size_t m = std::min(n - 1, A->src.size());
    memcpy(buf, A->src.data(), m);
    buf[m] = 0;
  }
  return (int)A->src.size();
}

}  // extern "C"

namespace {

// Load the code object on the current device once; returns the device or -1.
int ensure_loaded(cf_auto* A) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  std::lock_guard<std::mutex> lk(A->mu);
  if (!A->mod[dev]) {
    hipModule_t m = nullptr;
    if (hipModuleLoadData(&m, A->code.data()) != hipSuccess) return -1;
    hipFunction_t fv = nullptr, fs = nullptr;
    if (hipModuleGetFunction(&fv, m, (A->name + "_vec").c_str()) != hipSuccess ||
        hipModuleGetFunction(&fs, m, (A->name + "_scalar").c_str()) != hipSuccess) {
      (void)hipModuleUnload(m);
      return -1;
    }
    A->mod[dev] = m;
    A->fn_vec[dev] = fv;
    A->fn_scalar[dev] = fs;
  }
  return dev;
}

// Global scheme: rows per round for the kernel form that runs (vector or
// scalar: their register use, and so their residency, differ), with every
// member workgroup of a round resident at once; an error if not even one
// row's members fit.
cf_status global_rows_per_round(cf_auto* A, int dev, bool vec, int64_t* rg) {
  int occ = 0, cus = 0;
  if (hipModuleOccupancyMaxActiveBlocksPerMultiprocessor(&occ, vec ? A->fn_vec[dev] : A->fn_scalar[dev], A->wg, 0) !=
          hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return CF_EHIP;
  const int64_t cap = (int64_t)occ * cus;
  *rg = std::min<int64_t>({A->rows, cap / A->members, kJoinWords});
  return *rg >= 1 ? CF_OK : CF_EOCCUPANCY;
}

// Workspace bytes of a Global launch: the partials of the larger round of the
// two kernel forms.
cf_status global_ws_bytes(cf_auto* A, int dev, size_t* bytes) {
  int64_t rv = 0, rs = 0;
  cf_status st = global_rows_per_round(A, dev, true, &rv);
  if (st == CF_OK) st = global_rows_per_round(A, dev, false, &rs);
  if (st != CF_OK) return st;
  *bytes = kSlotsOff + (size_t)std::max(rv, rs) * 2 * A->reductions * A->members * 8;
  return CF_OK;
}

}  // namespace

extern "C" {

size_t cf_auto_workspace_bytes(cf_auto* A) {
  if (!A) return (size_t)-1;
  if (!A->global || A->reductions == 0) return 0;  // no cross-workgroup exchange
  const int dev = ensure_loaded(A);
  if (dev < 0) return (size_t)-1;
  size_t bytes = 0;
  return global_ws_bytes(A, dev, &bytes) == CF_OK ? bytes : (size_t)-1;
}

cf_status cf_auto_launch(cf_auto* A, const void* const* args, int nargs, float* out, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  if (!A || !out || nargs < 0 || (nargs > 0 && !args)) return CF_EINVAL;
  struct {
    const float* p[kMaxSlots];
    float* out;
    long rows, cols;
    unsigned* err;
    unsigned long long* joins;
    unsigned long long* slots;
    int S, RG;
  } ka{};
  const size_t tile_bytes = (size_t)A->rows * (size_t)A->cols * 4;
  bool vec = A->cols % 4 == 0 && aligned16(out);
  for (size_t i = 0; i < A->g.size(); ++i) {
    const int op = A->g[i].op;
    if (!A->live[i] || (op != CF_G_INPUT && op != CF_G_ROWVEC && op != CF_G_COLVEC)) continue;
    const int s = A->g[i].slot;
    if (s >= nargs || !args[s]) return CF_EINVAL;
    const size_t bytes = op == CF_G_INPUT ? tile_bytes : (size_t)(op == CF_G_ROWVEC ? A->cols : A->rows) * 4;
    if (overlap(out, tile_bytes, args[s], bytes)) return CF_EINVAL;
    if (op != CF_G_COLVEC) vec = vec && aligned16(args[s]);
    ka.p[s] = static_cast<const float*>(args[s]);
  }
  const bool exch = A->global && A->reductions > 0;  // members exchange partials through ws
  if (exch && (!ws || overlap(ws, ws_bytes, out, tile_bytes))) return !ws ? CF_EWORKSPACE : CF_EINVAL;
  ka.out = out;
  ka.rows = (long)A->rows;
  ka.cols = (long)A->cols;
  const int dev = ensure_loaded(A);
  if (dev < 0) return CF_EHIP;
  unsigned grid = 0;
  if (A->global) {
    int64_t rg = 0;
    size_t need = 0;
    cf_status st = global_rows_per_round(A, dev, vec, &rg);
    if (st == CF_OK && exch) st = global_ws_bytes(A, dev, &need);
    if (st != CF_OK) return st;
    if (exch) {
      if (ws_bytes < need) return CF_EWORKSPACE;
      char* base = static_cast<char*>(ws);
      ka.err = reinterpret_cast<unsigned*>(base);
      ka.joins = reinterpret_cast<unsigned long long*>(base + 256);
      ka.slots = reinterpret_cast<unsigned long long*>(base + kSlotsOff);
    }
    ka.S = A->members;
    ka.RG = (int)rg;
    grid = (unsigned)(rg * A->members);
  } else {
    const int64_t blocks = (A->rows + A->rows_per_wg - 1) / A->rows_per_wg;
    // a grid-stride launch of at most 32 workgroups of 256 lanes per CU (by lanes)
    const int64_t cap = (int64_t)8192 * 256 / A->wg;
    grid = (unsigned)std::min<int64_t>(blocks, cap);
  }
  void* params[] = {&ka};
  const hipError_t e = hipModuleLaunchKernel(vec ? A->fn_vec[dev] : A->fn_scalar[dev], grid, 1, 1, (unsigned)A->wg, 1,
                                             1, 0, stream, params, nullptr);
  return e == hipSuccess ? CF_OK : CF_EHIP;
}

void cf_auto_free(cf_auto* A) {
  if (!A) return;
  for (int d = 0; d < kMaxDevices; ++d)
    if (A->mod[d]) (void)hipModuleUnload(A->mod[d]);
  delete A;
}

}  // extern "C"
