// Fusion Spec IR: Phi (captured graph -> nested S) and Psi (S -> one of the
// library's precompiled stitched kernels, with its arguments bound).
//
// [ComFuse] Frontend / Fusion Spec IR (eq. 9 and 10, the Phi patterns, the
// recursive split at Reduction nodes, Psi's structural traversal).  Host
// code only: nothing here touches the device except cf_spec_launch, which
// calls the matched C-ABI entry point.

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "cf.h"
#include "cf_spec.h"

namespace {

constexpr int kMaxNodes = 256;

// Node categories of S: accumulator entry, broadcasts, element-wise
// computation and reduction (eq. 10), the element-wise read of a 2-D
// placeholder, and the entry placeholders of a nested S.
enum Cat {
  kAcc,      // the root: MatMul accumulator, or the input tile of a memory-intensive subgraph
  kLoad,     // a 2-D placeholder read elementwise (residual)
  kBRow,     // row-vector broadcast of a length-cols placeholder
  kBCol,     // column broadcast of a per-row value
  kBScalar,  // scalar broadcast of a constant
  kColVec,   // a per-row placeholder read as a per-row value
  kCompute,  // element-wise computation, on tiles or on per-row values
  kReduce,   // row reduction; it ends its level
  kStat,     // nested-S entry: the enclosing level's reduction statistic
  kPass,     // nested-S entry: a value of an enclosing level read again
};
const char* cat_name(int c) {
  static const char* n[] = {"acc", "load", "bcast_row", "bcast_col", "bcast_scalar", "colvec", "compute", "reduce",
                            "stat", "pass"};
  return n[c];
}
const char* op_name(int op) {
  static const char* n[] = {"input", "operand", "matmul", "rowvec", "colvec", "tensor", "const",
                            "add", "sub", "mul", "div", "pow", "exp", "square", "rsqrt", "relu",
                            "gelu_tanh", "silu", "rowsum", "rowmax"};
  return op >= 0 && op <= CF_G_ROWMAX ? n[op] : "-";
}
bool is_binary(int op) { return op >= CF_G_ADD && op <= CF_G_POW; }
bool is_unary(int op) { return op >= CF_G_EXP && op <= CF_G_SILU; }
bool is_reduce(int op) { return op == CF_G_ROWSUM || op == CF_G_ROWMAX; }
bool is_placeholder(int op) {
  return op == CF_G_INPUT || op == CF_G_OPERAND || op == CF_G_ROWVEC || op == CF_G_COLVEC || op == CF_G_TENSOR;
}
bool commutes(int op) { return op == CF_G_ADD || op == CF_G_MUL; }

// Shape class of a graph value.
enum Shape { kTile, kRowVal, kVec, kScalar };

struct SNode {
  int cat = kCompute;
  int op = -1;          // cf_gop: computation, reduction, placeholder or root kind
  int in[2] = {-1, -1};  // S inputs (entries: the enclosing-level node they stand for)
  int level = 0;
  int src = -1;         // graph node this S node stands for
  int attr = 0;         // MatMul operand layout
  int slot = -1;        // placeholders: argument slot
  double value = 0;     // constants
};

struct Param {
  int slot, op, node;  // argument slot, placeholder kind, graph node
};

// Argument roles of the precompiled kernels, and roles of their constants.
enum Role { kRX, kRA, kRW, kRBias, kRR, kRGamma, kRBeta, kRV, kNumRoles };
enum CRole { kCLit, kCCols, kCEps, kCP, kCScale, kNumCRoles };
const char* role_name(int r) {
  static const char* n[] = {"x", "A", "W", "bias", "R", "gamma", "beta", "v"};
  return n[r];
}
const char* crole_name(int r) {
  static const char* n[] = {"literal", "cols", "eps", "p", "scale"};
  return n[r];
}

// The stage DAGs the library implements.
enum Family {
  kFSoftmax, kFLayerNorm, kFLayerNormAffine, kFRmsNorm, kFRmsNormGain, kFPowSoftmax, kFGemmLN, kFGemmLNNoRes,
  kFGemmSoftmax, kFGemmAct0,  // + 2 * act index + has_bias, act index 0..5 (none, relu, gelu, silu, square, rsqrt)
  kNumFamilies = kFGemmAct0 + 12
};
const int kActOps[6] = {-1, CF_G_RELU, CF_G_GELU_TANH, CF_G_SILU, CF_G_SQUARE, CF_G_RSQRT};
const int kActIds[6] = {CF_ACT_NONE, CF_ACT_RELU, CF_ACT_GELU_TANH, CF_ACT_SILU, CF_ACT_SQUARE, CF_ACT_RSQRT};

}  // namespace

struct cf_spec {
  int64_t rows = 0, cols = 0, k = 0;
  std::vector<SNode> s;       // level by level, each level in topological order
  std::vector<int> tau;       // per level: its terminal (the reduction, except in the last level)
  std::vector<Param> params;  // the runtime parameter table A
  std::string signature;
  // Psi's match
  int family = -1;
  int role_slot[kNumRoles];
  double role_const[kNumCRoles];
};

namespace {

// ------------------------------------------------------------------- Phi

struct Lowering {
  const cf_gnode* g = nullptr;
  int n = 0;
  std::vector<int> level;  // value level (-1: placeholder or constant, read wherever used)
  std::vector<int> shape;
  std::vector<int> s_of;   // graph node -> the S node that computes it
  std::vector<std::vector<std::pair<int, int>>> entry;  // per level: (graph node, entry S node)
  cf_spec* sp = nullptr;
};

// Level at which graph value j can be read (a statistic one past its reduction).
int avail(const Lowering& L, int j) { return L.level[j] + (is_reduce(L.g[j].op) ? 1 : 0); }

cf_status infer(Lowering& L) {
  const cf_gnode* g = L.g;
  L.shape.assign(L.n, -1);
  L.level.assign(L.n, -1);
  for (int i = 0; i < L.n; ++i) {
    const int op = g[i].op;
    auto in_ok = [&](int j) { return j >= 0 && j < i; };
    if (is_placeholder(op) || op == CF_G_CONST) {
      if (g[i].in0 != -1 || g[i].in1 != -1) return CF_EINVAL;
      if (is_placeholder(op) && g[i].slot < 0) return CF_EINVAL;
      L.shape[i] = op == CF_G_ROWVEC ? kVec : op == CF_G_COLVEC ? kRowVal : op == CF_G_CONST ? kScalar : kTile;
      if (op == CF_G_INPUT) L.level[i] = 0;
      continue;
    }
    if (op == CF_G_MATMUL) {
      if (!in_ok(g[i].in0) || !in_ok(g[i].in1) || g[i].attr < 0 || g[i].attr > 1) return CF_EINVAL;
      if (g[g[i].in0].op != CF_G_OPERAND || g[g[i].in1].op != CF_G_OPERAND) return CF_EUNSUPPORTED;
      L.shape[i] = kTile;
      L.level[i] = 0;
      continue;
    }
    const int ni = is_binary(op) ? 2 : 1;
    const int in[2] = {g[i].in0, g[i].in1};
    if (!in_ok(in[0]) || (ni == 2 ? !in_ok(in[1]) : in[1] != -1)) return CF_EINVAL;
    for (int q = 0; q < ni; ++q)
      if (g[in[q]].op == CF_G_OPERAND) return CF_EUNSUPPORTED;  // an operand feeds its MatMul only
    int lv = 0;
    for (int q = 0; q < ni; ++q)
      if (L.level[in[q]] >= 0) lv = std::max(lv, avail(L, in[q]));
    L.level[i] = lv;
    const int sa = L.shape[in[0]];
    if (is_reduce(op)) {
      if (sa != kTile) return CF_EUNSUPPORTED;  // a reduction runs over the rows of a tile
      L.shape[i] = kRowVal;
    } else if (is_unary(op)) {
      if (sa != kTile && sa != kRowVal) return CF_EUNSUPPORTED;  // parameters are read, not transformed
      L.shape[i] = sa;
    } else {
      const int sb = L.shape[in[1]];
      if (op == CF_G_POW && sb != kScalar) return CF_EUNSUPPORTED;
      const bool da = sa == kTile || sa == kRowVal, db = sb == kTile || sb == kRowVal;
      if (!da && !db) return CF_EUNSUPPORTED;  // arithmetic on parameters alone
      if ((sa == kVec && sb != kTile) || (sb == kVec && sa != kTile)) return CF_EUNSUPPORTED;
      L.shape[i] = (sa == kTile || sb == kTile) ? kTile : kRowVal;
    }
  }
  return CF_OK;
}

int add_s(cf_spec* sp, SNode n) {
  sp->s.push_back(n);
  return (int)sp->s.size() - 1;
}

// The S node through which level `lv` reads graph value j as shape `want`:
// a broadcast for a constant or a 1-D placeholder, an element-wise load for
// a 2-D placeholder, the value itself within its own level, else an entry
// of this level (the statistic of the enclosing reduction, or a
// passthrough), then a column broadcast when a per-row value meets a tile.
int read_value(Lowering& L, int j, int lv, int want) {
  const cf_gnode* g = L.g;
  cf_spec* sp = L.sp;
  const int op = g[j].op;
  SNode b;
  b.level = lv;
  b.src = j;
  b.op = op;
  b.slot = g[j].slot;
  if (op == CF_G_CONST) {
    b.cat = kBScalar;
    b.slot = -1;
    b.value = g[j].value;
    return add_s(sp, b);
  }
  if (op == CF_G_ROWVEC) {
    b.cat = kBRow;
    return add_s(sp, b);
  }
  if (op == CF_G_TENSOR) {
    b.cat = kLoad;
    return add_s(sp, b);
  }
  int inner;
  if (op == CF_G_COLVEC) {
    b.cat = kColVec;
    inner = add_s(sp, b);
  } else if (avail(L, j) == lv && !is_reduce(op)) {
    inner = L.s_of[j];
  } else {
    inner = -1;
    for (auto& e : L.entry[lv])
      if (e.first == j) inner = e.second;
    if (inner < 0) {
      SNode e;
      e.level = lv;
      e.src = j;
      e.cat = (is_reduce(op) && avail(L, j) == lv) ? kStat : kPass;
      e.op = e.cat == kStat ? op : -1;
      e.in[0] = L.s_of[j];
      inner = add_s(sp, e);
      L.entry[lv].push_back({j, inner});
    }
  }
  if (want == kTile && L.shape[j] == kRowVal) {
    SNode c;
    c.cat = kBCol;
    c.level = lv;
    c.src = j;
    c.in[0] = inner;
    return add_s(sp, c);
  }
  return inner;
}

void mark_live(const cf_gnode* g, int t, std::vector<char>& live) {
  if (t < 0 || live[t]) return;
  live[t] = 1;
  if (g[t].op == CF_G_CONST || is_placeholder(g[t].op)) return;
  mark_live(g, g[t].in0, live);
  mark_live(g, g[t].in1, live);
}

cf_status phi(const cf_gnode* g, int n, int terminal, cf_spec* sp) {
  if (!g || n <= 0 || n > kMaxNodes || terminal < 0 || terminal >= n) return CF_EINVAL;
  for (int i = 0; i < n; ++i)
    if (g[i].op < CF_G_INPUT || g[i].op > CF_G_ROWMAX) return CF_EINVAL;
  Lowering L;
  L.g = g;
  L.n = n;
  L.sp = sp;
  cf_status st = infer(L);
  if (st != CF_OK) return st;
  std::vector<char> live(n, 0);
  mark_live(g, terminal, live);
  // one root among the nodes the output depends on: a MatMul, or one input tile
  int root = -1, roots = 0;
  for (int i = 0; i < n; ++i)
    if (live[i] && (g[i].op == CF_G_MATMUL || g[i].op == CF_G_INPUT)) {
      root = i;
      ++roots;
    }
  if (roots != 1 || L.shape[terminal] != kTile) return CF_EUNSUPPORTED;
  // levels: every level but the last ends in exactly one reduction
  const int nlev = L.level[terminal] + 1;
  std::vector<int> red_at(nlev, -1);
  for (int i = 0; i < n; ++i) {
    if (!live[i] || L.level[i] < 0) continue;
    if (L.level[i] >= nlev) return CF_EUNSUPPORTED;
    if (is_reduce(g[i].op)) {
      if (red_at[L.level[i]] >= 0 || L.level[i] == nlev - 1) return CF_EUNSUPPORTED;
      red_at[L.level[i]] = i;
    }
  }
  for (int l = 0; l + 1 < nlev; ++l)
    if (red_at[l] < 0) return CF_EUNSUPPORTED;
  L.s_of.assign(n, -1);
  L.entry.assign(nlev, {});
  sp->tau.assign(nlev, -1);
  if (g[root].op == CF_G_INPUT) {
    SNode a;
    a.cat = kAcc;
    a.op = CF_G_INPUT;
    a.src = root;
    a.slot = g[root].slot;
    L.s_of[root] = add_s(sp, a);
    sp->params.push_back({g[root].slot, CF_G_INPUT, root});
  }
  for (int lv = 0; lv < nlev; ++lv) {
    for (int i = 0; i < n; ++i) {
      const int op = g[i].op;
      if (!live[i] || L.level[i] != lv || is_placeholder(op) || op == CF_G_CONST) continue;
      SNode s;
      s.level = lv;
      s.src = i;
      s.op = op;
      if (op == CF_G_MATMUL) {
        s.cat = kAcc;
        s.attr = g[i].attr;
        for (int o : {g[i].in0, g[i].in1}) sp->params.push_back({g[o].slot, CF_G_OPERAND, o});
      } else {
        s.cat = is_reduce(op) ? kReduce : kCompute;
        const int want = is_reduce(op) ? kTile : L.shape[i];
        s.in[0] = read_value(L, g[i].in0, lv, want);
        if (is_binary(op)) s.in[1] = read_value(L, g[i].in1, lv, want);
      }
      L.s_of[i] = add_s(sp, s);
      if (is_reduce(op)) sp->tau[lv] = L.s_of[i];
    }
  }
  sp->tau[nlev - 1] = L.s_of[terminal];
  if (sp->tau[nlev - 1] < 0) return CF_EUNSUPPORTED;  // the output is the input itself
  for (auto& s : sp->s)
    if (s.cat == kBRow || s.cat == kLoad || s.cat == kColVec) {
      bool seen = false;
      for (auto& p : sp->params) seen |= p.node == s.src;
      if (!seen) sp->params.push_back({s.slot, s.op, s.src});
    }
  return CF_OK;
}

// ------------------------------------------------------------------- Psi

// Canonical form of the subtree at S node i: categories, operators and
// shape of the data flow, operands of commutative operators ordered by
// their own canonical forms; constants and placeholders appear by kind only.
struct Canon {
  const cf_spec* sp;
  std::vector<std::string> memo;
  explicit Canon(const cf_spec* s) : sp(s), memo(s->s.size()) {}
  const std::string& str(int i) {
    if (!memo[i].empty()) return memo[i];
    const SNode& n = sp->s[i];
    std::string r;
    switch (n.cat) {
      case kAcc: r = n.op == CF_G_MATMUL ? (n.attr ? "MM_NT" : "MM_NN") : "X"; break;
      case kLoad: r = "R"; break;
      case kBRow: r = "BR(V)"; break;
      case kBScalar: r = "C"; break;
      case kColVec: r = "CV"; break;
      case kBCol: r = "BC(" + str(n.in[0]) + ")"; break;
      case kStat: r = std::string("STAT(") + op_name(n.op) + ")"; break;
      case kPass: r = "PASS(" + str(n.in[0]) + ")"; break;
      case kReduce: r = std::string(op_name(n.op)) + "(" + str(n.in[0]) + ")"; break;
      default: {
        r = std::string(op_name(n.op)) + "(";
        if (n.in[1] < 0) {
          r += str(n.in[0]);
        } else {
          const std::string &a = str(n.in[0]), &b = str(n.in[1]);
          r += (commutes(n.op) && b < a) ? b + "," + a : a + "," + b;
        }
        r += ")";
      }
    }
    memo[i] = r;
    return memo[i];
  }
  // constants and placeholders (S nodes) in canonical order
  void leaves(int i, std::vector<int>& out) {
    const SNode& n = sp->s[i];
    switch (n.cat) {
      case kAcc:
      case kLoad:
      case kBRow:
      case kBScalar:
      case kColVec: out.push_back(i); return;
      case kStat: return;
      case kBCol:
      case kPass:
      case kReduce: leaves(n.in[0], out); return;
      default:
        if (n.in[1] < 0) {
          leaves(n.in[0], out);
        } else if (commutes(n.op) && str(n.in[1]) < str(n.in[0])) {
          leaves(n.in[1], out);
          leaves(n.in[0], out);
        } else {
          leaves(n.in[0], out);
          leaves(n.in[1], out);
        }
    }
  }
  std::string signature() {
    std::string r;
    for (size_t l = 0; l < sp->tau.size(); ++l) r += (l ? " ; " : "") + str(sp->tau[l]);
    return r;
  }
  std::vector<int> all_leaves() {
    std::vector<int> out;
    for (int t : sp->tau) leaves(t, out);
    return out;
  }
};

// Template graphs of the families, in the caller's node format: placeholder
// slots carry the argument role, constant attrs the constant's role.
struct GB {
  std::vector<cf_gnode> v;
  int add(int op, int a = -1, int b = -1, int attr = 0, int slot = -1) {
    cf_gnode n{};
    n.op = op;
    n.in0 = a;
    n.in1 = b;
    n.attr = attr;
    n.slot = slot;
    v.push_back(n);
    return (int)v.size() - 1;
  }
  int ph(int op, int role) { return add(op, -1, -1, 0, role); }
  int cst(int crole) { return add(CF_G_CONST, -1, -1, crole); }
};

int softmax_chain(GB& b, int t) {
  const int m = b.add(CF_G_ROWMAX, t);
  const int e = b.add(CF_G_EXP, b.add(CF_G_SUB, t, m));
  return b.add(CF_G_DIV, e, b.add(CF_G_ROWSUM, e));
}
int layernorm_chain(GB& b, int u, bool affine) {
  const int mu = b.add(CF_G_DIV, b.add(CF_G_ROWSUM, u), b.cst(kCCols));
  const int c = b.add(CF_G_SUB, u, mu);
  const int var = b.add(CF_G_DIV, b.add(CF_G_ROWSUM, b.add(CF_G_SQUARE, c)), b.cst(kCCols));
  int y = b.add(CF_G_MUL, c, b.add(CF_G_RSQRT, b.add(CF_G_ADD, var, b.cst(kCEps))));
  if (affine) y = b.add(CF_G_ADD, b.add(CF_G_MUL, y, b.ph(CF_G_ROWVEC, kRGamma)), b.ph(CF_G_ROWVEC, kRBeta));
  return y;
}

GB family_graph(int f) {
  GB b;
  if (f <= kFPowSoftmax) {
    const int x = b.ph(CF_G_INPUT, kRX);
    switch (f) {
      case kFSoftmax: softmax_chain(b, x); break;
      case kFLayerNorm: layernorm_chain(b, x, false); break;
      case kFLayerNormAffine: layernorm_chain(b, x, true); break;
      case kFRmsNorm:
      case kFRmsNormGain: {
        const int ms = b.add(CF_G_DIV, b.add(CF_G_ROWSUM, b.add(CF_G_SQUARE, x)), b.cst(kCCols));
        int y = b.add(CF_G_MUL, x, b.add(CF_G_RSQRT, b.add(CF_G_ADD, ms, b.cst(kCEps))));
        if (f == kFRmsNormGain) y = b.add(CF_G_MUL, y, b.ph(CF_G_ROWVEC, kRGamma));
        break;
      }
      default: {
        const int pv = b.add(CF_G_POW, b.ph(CF_G_COLVEC, kRV), b.cst(kCP));
        softmax_chain(b, b.add(CF_G_ADD, x, pv));
      }
    }
    return b;
  }
  const int a = b.ph(CF_G_OPERAND, kRA), w = b.ph(CF_G_OPERAND, kRW);
  if (f == kFGemmSoftmax) {
    softmax_chain(b, b.add(CF_G_MUL, b.add(CF_G_MATMUL, a, w, 1), b.cst(kCScale)));
    return b;
  }
  int u = b.add(CF_G_MATMUL, a, w, 0);
  if (f == kFGemmLN || f == kFGemmLNNoRes) {
    u = b.add(CF_G_ADD, u, b.ph(CF_G_ROWVEC, kRBias));
    if (f == kFGemmLN) u = b.add(CF_G_ADD, u, b.ph(CF_G_TENSOR, kRR));
    layernorm_chain(b, u, true);
    return b;
  }
  const int act = (f - kFGemmAct0) / 2, bias = (f - kFGemmAct0) % 2;
  if (bias) u = b.add(CF_G_ADD, u, b.ph(CF_G_ROWVEC, kRBias));
  if (kActOps[act] >= 0) b.add(kActOps[act], u);
  return b;
}

struct FamilyForm {
  std::string sig;
  std::vector<SNode> leaves;  // the template's constants and placeholders, canonical order
};
const std::vector<FamilyForm>& family_forms() {
  static const std::vector<FamilyForm> forms = [] {
    std::vector<FamilyForm> r(kNumFamilies);
    for (int f = 0; f < kNumFamilies; ++f) {
      GB b = family_graph(f);
      cf_spec t;
      if (phi(b.v.data(), (int)b.v.size(), (int)b.v.size() - 1, &t) != CF_OK) continue;
      Canon c(&t);
      r[f].sig = c.signature();
      for (int i : c.all_leaves()) {
        SNode n = t.s[i];
        if (n.cat == kBScalar) n.attr = b.v[n.src].attr;  // the constant's role
        r[f].leaves.push_back(n);
      }
    }
    return r;
  }();
  return forms;
}

cf_status psi(cf_spec* sp) {
  Canon c(sp);
  sp->signature = c.signature();
  const std::vector<int> mine = c.all_leaves();
  const auto& forms = family_forms();
  for (int f = 0; f < kNumFamilies; ++f) {
    const FamilyForm& F = forms[f];
    if (F.sig.empty() || F.sig != sp->signature || F.leaves.size() != mine.size()) continue;
    int rs[kNumRoles];
    double rc[kNumCRoles];
    bool have_c[kNumCRoles] = {};
    std::fill(rs, rs + kNumRoles, -1);
    std::fill(rc, rc + kNumCRoles, 0.0);
    bool ok = true;
    for (size_t q = 0; q < mine.size() && ok; ++q) {
      const SNode& u = sp->s[mine[q]];
      const SNode& t = F.leaves[q];
      if (u.cat != t.cat) {
        ok = false;
      } else if (t.cat == kBScalar) {
        const int role = t.attr;
        if (!std::isfinite(u.value)) ok = false;
        else if (role == kCCols) ok = u.value == (double)sp->cols;
        else if (role == kCEps && u.value < 0.0) ok = false;
        if (ok && role != kCCols) {
          if (have_c[role] && rc[role] != u.value) ok = false;  // one role, one value
          rc[role] = u.value;
          have_c[role] = true;
        }
      } else if (t.cat == kAcc && t.op == CF_G_MATMUL) {
        // the operands are bound from the MatMul node itself, in its input order
      } else {
        const int role = t.slot;
        if (rs[role] >= 0 && rs[role] != u.slot) ok = false;
        rs[role] = u.slot;
      }
    }
    if (!ok) continue;
    sp->family = f;
    std::copy(rs, rs + kNumRoles, sp->role_slot);
    std::copy(rc, rc + kNumCRoles, sp->role_const);
    return CF_OK;
  }
  return CF_EUNSUPPORTED;
}

const char* family_call(int f) {
  switch (f) {
    case kFSoftmax: return "cf_stitch_softmax";
    case kFLayerNorm: return "cf_stitch_layernorm";
    case kFLayerNormAffine: return "cf_stitch_layernorm_affine";
    case kFRmsNorm:
    case kFRmsNormGain: return "cf_stitch_rmsnorm";
    case kFPowSoftmax: return "cf_stitch_pow_bcast_add";
    case kFGemmLN:
    case kFGemmLNNoRes: return "cf_gemm_ln";
    case kFGemmSoftmax: return "cf_gemm_softmax";
  }
  return "cf_gemm_act";
}

int family_op(int f) {
  switch (f) {
    case kFSoftmax: return CF_OP_STITCH_SOFTMAX;
    case kFLayerNorm: return CF_OP_STITCH_LAYERNORM;
    case kFLayerNormAffine: return CF_OP_STITCH_LAYERNORM_AFFINE;
    case kFRmsNorm:
    case kFRmsNormGain: return CF_OP_STITCH_RMSNORM;
    case kFPowSoftmax: return CF_OP_STITCH_POW_BCAST_ADD;
    case kFGemmLN:
    case kFGemmLNNoRes: return CF_OP_GEMM_LN;
    case kFGemmSoftmax: return CF_OP_GEMM_SOFTMAX;
  }
  return CF_OP_GEMM_ACT;
}

bool family_is_gemm(int f) { return f >= kFGemmLN; }

}  // namespace

extern "C" {

cf_status cf_spec_build(const cf_gnode* nodes, int n, int terminal, int64_t rows, int64_t cols, int64_t k,
                        cf_spec** out) {
  if (!out) return CF_EINVAL;
  *out = nullptr;
  if (rows <= 0 || cols <= 0 || k < 0) return CF_EINVAL;
  cf_spec* sp = new cf_spec;
  sp->rows = rows;
  sp->cols = cols;
  sp->k = k;
  cf_status st = phi(nodes, n, terminal, sp);
  if (st == CF_OK) {
    // the MatMul operands are bound by their position in the MatMul node
    st = psi(sp);
  }
  if (st == CF_OK) {
    const bool gemm = family_is_gemm(sp->family);
    if (gemm != (k > 0)) st = CF_EINVAL;  // a MatMul root needs its reduction depth, and only it
    if (gemm) {
      for (const SNode& s : sp->s)
        if (s.cat == kAcc && s.op == CF_G_MATMUL) {
          sp->role_slot[kRA] = nodes[nodes[s.src].in0].slot;
          sp->role_slot[kRW] = nodes[nodes[s.src].in1].slot;
        }
    }
  }
  if (st != CF_OK) {
    delete sp;
    return st;
  }
  *out = sp;
  return CF_OK;
}

int cf_spec_describe(const cf_spec* sp, char* buf, size_t n) {
  if (!sp) return -1;
  std::string j = "{\"rows\":" + std::to_string(sp->rows) + ",\"cols\":" + std::to_string(sp->cols) +
                  ",\"k\":" + std::to_string(sp->k) + ",\"levels\":[";
  char tmp[160];
  for (size_t l = 0; l < sp->tau.size(); ++l) {
    j += (l ? "," : "");
    j += "{\"level\":" + std::to_string(l) + ",\"tau\":" + std::to_string(sp->tau[l]) + ",\"nodes\":[";
    bool first = true;
    for (size_t i = 0; i < sp->s.size(); ++i) {
      const SNode& s = sp->s[i];
      if (s.level != (int)l) continue;
      snprintf(tmp, sizeof tmp, "%s{\"id\":%zu,\"cat\":\"%s\",\"op\":\"%s\",\"in\":[%d,%d],\"src\":%d", first ? "" : ",",
               i, cat_name(s.cat), op_name(s.op), s.in[0], s.in[1], s.src);
      j += tmp;
      if (s.cat == kBScalar) {
        snprintf(tmp, sizeof tmp, ",\"value\":%.17g", s.value);
        j += tmp;
      }
      if (s.slot >= 0) j += ",\"slot\":" + std::to_string(s.slot);
      j += "}";
      first = false;
    }
    j += "]}";
  }
  j += "],\"depth\":" + std::to_string(sp->tau.size()) + ",\"params\":[";
  for (size_t p = 0; p < sp->params.size(); ++p) {
    snprintf(tmp, sizeof tmp, "%s{\"slot\":%d,\"kind\":\"%s\",\"node\":%d}", p ? "," : "", sp->params[p].slot,
             op_name(sp->params[p].op), sp->params[p].node);
    j += tmp;
  }
  j += "],\"signature\":\"" + sp->signature + "\",\"match\":{\"call\":\"" + family_call(sp->family) + "\"";
  if (sp->family >= kFGemmAct0) {
    const int act = (sp->family - kFGemmAct0) / 2;
    j += std::string(",\"act\":\"") + (kActOps[act] < 0 ? "none" : op_name(kActOps[act])) + "\"";
  }
  j += ",\"args\":{";
  bool first = true;
  for (int r = 0; r < kNumRoles; ++r)
    if (sp->role_slot[r] >= 0) {
      j += std::string(first ? "" : ",") + "\"" + role_name(r) + "\":" + std::to_string(sp->role_slot[r]);
      first = false;
    }
  j += "},\"constants\":{";
  first = true;
  for (int r = kCEps; r < kNumCRoles; ++r) {
    const int f = sp->family;
    const bool used = (r == kCEps && (f == kFLayerNorm || f == kFLayerNormAffine || f == kFRmsNorm ||
                                      f == kFRmsNormGain || f == kFGemmLN || f == kFGemmLNNoRes)) ||
                      (r == kCP && f == kFPowSoftmax) || (r == kCScale && f == kFGemmSoftmax);
    if (!used) continue;
    snprintf(tmp, sizeof tmp, "%s\"%s\":%.17g", first ? "" : ",", crole_name(r), sp->role_const[r]);
    j += tmp;
    first = false;
  }
  j += "}}}";
  if (buf && n > 0) {
    const size_t m = std::min(n - 1, j.size());
    memcpy(buf, j.data(), m);
    buf[m] = 0;
  }
  return (int)j.size();
}

size_t cf_spec_workspace_bytes(const cf_spec* sp) {
  if (!sp) return (size_t)-1;
  return cf_workspace_bytes(family_op(sp->family), sp->rows, sp->cols, sp->k);
}

cf_status cf_spec_launch(const cf_spec* sp, const void* const* args, int nargs, void* out, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  if (!sp || !out || (!args && nargs > 0) || nargs < 0) return CF_EINVAL;
  const void* a[kNumRoles] = {};
  for (int r = 0; r < kNumRoles; ++r) {
    const int s = sp->role_slot[r];
    if (s < 0) continue;
    if (s >= nargs || !args[s]) return CF_EINVAL;
    a[r] = args[s];
  }
  const int64_t M = sp->rows, N = sp->cols, K = sp->k;
  const float eps = (float)sp->role_const[kCEps];
  auto X = static_cast<const float*>(a[kRX]);
  auto F = [&](int r) { return static_cast<const float*>(a[r]); };
  auto B = [&](int r) { return static_cast<const cf_bf16*>(a[r]); };
  float* y = static_cast<float*>(out);
  cf_bf16* Y = static_cast<cf_bf16*>(out);
  switch (sp->family) {
    case kFSoftmax: return cf_stitch_softmax(X, y, M, N, ws, ws_bytes, stream);
    case kFLayerNorm: return cf_stitch_layernorm(X, y, M, N, eps, ws, ws_bytes, stream);
    case kFLayerNormAffine:
      return cf_stitch_layernorm_affine(X, F(kRGamma), F(kRBeta), y, M, N, eps, ws, ws_bytes, stream);
    case kFRmsNorm: return cf_stitch_rmsnorm(X, nullptr, y, M, N, eps, ws, ws_bytes, stream);
    case kFRmsNormGain: return cf_stitch_rmsnorm(X, F(kRGamma), y, M, N, eps, ws, ws_bytes, stream);
    case kFPowSoftmax:
      return cf_stitch_pow_bcast_add(X, F(kRV), (float)sp->role_const[kCP], y, nullptr, M, N, ws, ws_bytes, stream);
    case kFGemmLN:
    case kFGemmLNNoRes:
      return cf_gemm_ln(B(kRA), B(kRW), F(kRBias), sp->family == kFGemmLN ? B(kRR) : nullptr, F(kRGamma), F(kRBeta),
                        eps, Y, M, N, K, ws, ws_bytes, stream);
    case kFGemmSoftmax:
      return cf_gemm_softmax(B(kRA), B(kRW), (float)sp->role_const[kCScale], Y, M, N, K, ws, ws_bytes, stream);
  }
  if (sp->family >= kFGemmAct0 && sp->family < kNumFamilies) {
    const int act = (sp->family - kFGemmAct0) / 2, bias = (sp->family - kFGemmAct0) % 2;
    return cf_gemm_act(B(kRA), B(kRW), bias ? F(kRBias) : nullptr, kActIds[act], Y, M, N, K, ws, ws_bytes, stream);
  }
  return CF_EINVAL;
}

void cf_spec_free(cf_spec* sp) { delete sp; }

}  // extern "C"
