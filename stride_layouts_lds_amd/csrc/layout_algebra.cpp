// layout_algebra.cpp -- the host layout algebra (see layout_algebra.hpp).
#include "layout_algebra.hpp"

#include <algorithm>
#include <numeric>

namespace sl {
namespace la {
namespace {

// Checked arithmetic: results stay below 2^62, beyond which an operation is
// reported as undefined rather than wrapping.
constexpr int64_t kLimit = int64_t(1) << 62;
int64_t mul(int64_t a, int64_t b) {
  int64_t r;
  if (__builtin_mul_overflow(a, b, &r) || r > kLimit || r < -kLimit) throw Error{"integer overflow"};
  return r;
}
int64_t add(int64_t a, int64_t b) {
  int64_t r;
  if (__builtin_add_overflow(a, b, &r) || r > kLimit || r < -kLimit) throw Error{"integer overflow"};
  return r;
}

// ------------------------------------------------------------- parsing

struct Cursor {
  const std::string& s;
  size_t i = 0;
  void ws() {
    while (i < s.size() && (s[i] == ' ' || s[i] == '\t')) ++i;
  }
  bool eat(char c) {
    ws();
    if (i < s.size() && s[i] == c) {
      ++i;
      return true;
    }
    return false;
  }
  void expect(char c) {
    if (!eat(c)) throw Error{std::string("expected '") + c + "' at position " + std::to_string(i) + " in \"" + s + "\""};
  }
  int64_t integer() {
    ws();
    size_t j = i;
    while (j < s.size() && s[j] >= '0' && s[j] <= '9') ++j;
    if (j == i) throw Error{"expected an integer at position " + std::to_string(i) + " in \"" + s + "\""};
    if (j - i > 18) throw Error{"integer too large in \"" + s + "\""};
    const int64_t v = std::stoll(s.substr(i, j - i));
    i = j;
    return v;
  }
};

// a tree of integers: "(a,(_b,c))" or "a"
struct Tree {
  bool leaf = true;
  int64_t v = 0;
  bool stat = false;
  std::vector<Tree> kids;
};

Tree parse_tree(Cursor& c, int depth = 0) {
  if (depth > 32) throw Error{"nesting too deep in \"" + c.s + "\""};
  Tree t;
  if (c.eat('(')) {
    t.leaf = false;
    do t.kids.push_back(parse_tree(c, depth + 1));
    while (c.eat(','));
    c.expect(')');
  } else {
    t.stat = c.eat('_');
    t.v = c.integer();
  }
  return t;
}

Layout zip(const Tree& shape, const Tree& stride) {
  if (shape.leaf != stride.leaf || shape.kids.size() != stride.kids.size())
    throw Error{"shape and stride trees differ"};
  if (shape.leaf) {
    Layout l = Layout::mode(shape.v, stride.v);
    l.shape_static = shape.stat;
    l.stride_static = stride.stat;
    return l;
  }
  std::vector<Layout> k;
  for (size_t i = 0; i < shape.kids.size(); ++i) k.push_back(zip(shape.kids[i], stride.kids[i]));
  return Layout::tuple(std::move(k));
}

Layout zeros_like(const Tree& shape) {
  if (shape.leaf) {
    Layout l = Layout::mode(shape.v, 0);
    l.shape_static = shape.stat;
    return l;
  }
  std::vector<Layout> k;
  for (const Tree& t : shape.kids) k.push_back(zeros_like(t));
  return Layout::tuple(std::move(k));
}

void tree_str(const Layout& l, std::string& out, bool stride, bool mark) {
  if (l.leaf) {
    if (mark && (stride ? l.stride_static : l.shape_static)) out += '_';
    out += std::to_string(stride ? l.stride : l.shape);
    return;
  }
  out += '(';
  for (size_t i = 0; i < l.kids.size(); ++i) {
    if (i) out += ',';
    tree_str(l.kids[i], out, stride, mark);
  }
  out += ')';
}

void flatten_into(const Layout& l, std::vector<Mode>& out) {
  if (l.leaf) {
    out.push_back({l.shape, l.stride, l.stride_static});
    return;
  }
  for (const Layout& k : l.kids) flatten_into(k, out);
}

Layout from_modes(const std::vector<Mode>& m) {
  if (m.empty()) return Layout::mode(1, 0);
  if (m.size() == 1) return Layout::mode(m[0].shape, m[0].stride, m[0].stat);
  std::vector<Layout> k;
  for (const Mode& x : m) k.push_back(Layout::mode(x.shape, x.stride, x.stat));
  return Layout::tuple(std::move(k));
}

// A (flat modes, coalesced) composed with the single mode s:d.  A's last mode
// is taken to continue past its extent (its stride keeps counting), as a
// layout's last mode does when it is indexed beyond its size.  Steps: divide
// the stride d out of A's leading shapes, then keep A's modes until their
// sizes make up s.
Layout compose_mode(const std::vector<Mode>& a, int64_t s, int64_t d, bool stat) {
  for (const Mode& m : a)
    if (m.shape == 0) throw Error{"composition: the layout has an empty mode"};
  if (s == 0) throw Error{"composition: an empty mode"};
  if (s == 1) return Layout::mode(1, 0, stat);
  if (d == 0) return Layout::mode(s, 0, stat);
  std::vector<Mode> out;
  int64_t r = d, rest = s;
  for (size_t i = 0; i < a.size() && rest > 1; ++i) {
    int64_t S = a[i].shape, D = a[i].stride;
    const bool last = i + 1 == a.size();
    if (r > 1) {
      if (last) {
        D = mul(D, r);
        r = 1;
      } else if (r % S == 0) {
        r /= S;
        continue;
      } else if (S % r == 0) {
        S /= r;
        D = mul(D, r);
        r = 1;
      } else {
        throw Error{"composition: stride " + std::to_string(d) + " does not divide the layout's shape"};
      }
    }
    if (last) {
      out.push_back({rest, D, stat});
      rest = 1;
    } else if (rest % S == 0) {
      out.push_back({S, D, stat});
      rest /= S;
    } else if (S % rest == 0) {
      out.push_back({rest, D, stat});
      rest = 1;
    } else {
      throw Error{"composition: shape " + std::to_string(s) + " does not divide the layout's shape"};
    }
  }
  return coalesce(from_modes(out));
}

Layout compose_tree(const std::vector<Mode>& a, bool a_static, const Layout& b) {
  if (!b.leaf) {
    std::vector<Layout> k;
    for (const Layout& x : b.kids) k.push_back(compose_tree(a, a_static, x));
    return Layout::tuple(std::move(k));
  }
  return compose_mode(a, b.shape, b.stride, a_static && b.stride_static);
}

Layout map_leaves(const Layout& l, const std::vector<int64_t>& strides, size_t& at) {
  if (l.leaf) {
    Layout m = Layout::mode(l.shape, strides[at++]);
    m.shape_static = l.shape_static;
    return m;
  }
  std::vector<Layout> k;
  for (const Layout& x : l.kids) k.push_back(map_leaves(x, strides, at));
  return Layout::tuple(std::move(k));
}

// compact strides for the flat shapes `m`, taken in the order `idx`;
// size-1 modes get 0
std::vector<int64_t> compact_in_order(const std::vector<Mode>& m, const std::vector<size_t>& idx) {
  std::vector<int64_t> strides(m.size(), 0);
  int64_t cur = 1;
  for (size_t i : idx) {
    if (m[i].shape == 1) continue;
    strides[i] = cur;
    cur = mul(cur, m[i].shape);
  }
  return strides;
}

Layout tuple_of_modes(const Layout& l, size_t from) {
  std::vector<Layout> k;
  for (size_t i = from; i < l.rank(); ++i) k.push_back(l.at(i));
  return Layout::tuple(std::move(k));
}

}  // namespace

// ---------------------------------------------------------------- basics

Layout parse(const std::string& text) {
  Cursor c{text};
  Tree shape = parse_tree(c);
  c.expect(':');
  Tree stride = parse_tree(c);
  c.ws();
  if (c.i != text.size()) throw Error{"trailing text in \"" + text + "\""};
  return zip(shape, stride);
}

Layout parse_shape(const std::string& text) {
  Cursor c{text};
  Tree shape = parse_tree(c);
  c.ws();
  if (c.i != text.size()) throw Error{"trailing text in \"" + text + "\""};
  return zeros_like(shape);
}

std::string to_string(const Layout& l, bool mark_static) {
  std::string out;
  tree_str(l, out, false, mark_static);
  out += ':';
  tree_str(l, out, true, mark_static);
  return out;
}

std::vector<Mode> flatten(const Layout& l) {
  std::vector<Mode> out;
  flatten_into(l, out);
  return out;
}

int64_t size(const Layout& l) {
  int64_t n = 1;
  for (const Mode& m : flatten(l)) n = mul(n, m.shape);
  return n;
}

int64_t cosize(const Layout& l) {
  int64_t hi = 0;
  for (const Mode& m : flatten(l)) {
    if (m.shape == 0) return 0;
    hi = add(hi, mul(m.shape - 1, m.stride));
  }
  return add(hi, 1);
}

int64_t eval(const Layout& l, int64_t index) {
  int64_t off = 0;
  for (const Mode& m : flatten(l)) {
    if (m.shape == 0) return 0;
    off = add(off, mul(index % m.shape, m.stride));
    index /= m.shape;
  }
  return off;
}

bool all_static(const Layout& l) {
  if (l.leaf) return l.stride_static;
  for (const Layout& k : l.kids)
    if (!all_static(k)) return false;
  return true;
}

Layout coalesce(const Layout& l) {
  std::vector<Mode> out;
  for (const Mode& m : flatten(l)) {
    if (m.shape == 1) continue;
    if (!out.empty() && mul(out.back().shape, out.back().stride) == m.stride) {
      out.back().shape = mul(out.back().shape, m.shape);
      out.back().stat = out.back().stat && m.stat;
      continue;
    }
    out.push_back(m);
  }
  return from_modes(out);
}

Layout composition(const Layout& a, const Layout& b) {
  return compose_tree(flatten(coalesce(a)), all_static(a), b);
}

Layout complement(const Layout& a, int64_t cosize_target) {
  const bool stat = all_static(a);
  std::vector<Mode> m;
  for (const Mode& x : flatten(a))
    if (x.shape > 1 && x.stride > 0) m.push_back(x);
  std::stable_sort(m.begin(), m.end(), [](const Mode& x, const Mode& y) { return x.stride < y.stride; });
  std::vector<Mode> out;
  int64_t cur = 1;
  for (const Mode& x : m) {
    if (x.stride % cur != 0) throw Error{"complement: strides are not nested multiples"};
    if (x.stride / cur > 1) out.push_back({x.stride / cur, cur, stat});
    cur = mul(x.shape, x.stride);
  }
  const int64_t rest = cosize_target / cur + (cosize_target % cur != 0);
  if (rest > 1) out.push_back({rest, cur, stat});
  return coalesce(from_modes(out));
}

Layout right_inverse(const Layout& a) {
  const bool stat = all_static(a);
  const std::vector<Mode> m = flatten(a);
  struct Item {
    int64_t shape, stride, dom;
  };
  std::vector<Item> it;
  int64_t dom = 1;
  for (const Mode& x : m) {
    if (x.shape > 1 && x.stride > 0) it.push_back({x.shape, x.stride, dom});
    dom = mul(dom, x.shape);
  }
  std::stable_sort(it.begin(), it.end(), [](const Item& x, const Item& y) { return x.stride < y.stride; });
  std::vector<Mode> out;
  int64_t expect = 1;
  for (const Item& x : it) {
    if (x.stride != expect) break;  // the inverse covers the contiguous prefix of the image
    out.push_back({x.shape, x.dom, stat});
    expect = mul(expect, x.shape);
  }
  return coalesce(from_modes(out));
}

Layout zipped_divide(const Layout& a, const Layout& tiler) {
  if (a.rank() != tiler.rank())
    throw Error{"zipped_divide: the tiler needs one mode per mode of the layout"};
  std::vector<Layout> tiles, rests;
  for (size_t i = 0; i < a.rank(); ++i) {
    const Layout& t = tiler.at(i);
    const Layout div = composition(a.at(i), Layout::tuple({t, complement(t, size(a.at(i)))}));
    tiles.push_back(div.kids[0]);
    rests.push_back(div.kids[1]);
  }
  return Layout::tuple({Layout::tuple(std::move(tiles)), Layout::tuple(std::move(rests))});
}

Layout filter_zeros(const Layout& a) {
  if (a.leaf) {
    Layout l = a;
    if (a.stride_static && a.stride == 0) l.shape = 1;
    return l;
  }
  std::vector<Layout> k;
  for (const Layout& y : a.kids) k.push_back(filter_zeros(y));
  return Layout::tuple(std::move(k));
}

Layout compact_left(const Layout& a) {
  const std::vector<Mode> m = flatten(a);
  std::vector<size_t> idx(m.size());
  std::iota(idx.begin(), idx.end(), 0);
  const std::vector<int64_t> strides = compact_in_order(m, idx);
  size_t at = 0;
  return map_leaves(a, strides, at);
}

Layout make_ordered(const Layout& shape, const Layout& order) {
  const std::vector<Mode> m = flatten(shape), o = flatten(order);
  if (o.size() != m.size()) throw Error{"make_ordered: one order value per mode"};
  std::vector<size_t> stat, dyn;
  for (size_t i = 0; i < o.size(); ++i) (o[i].stat ? stat : dyn).push_back(i);
  std::stable_sort(stat.begin(), stat.end(), [&](size_t x, size_t y) { return o[x].stride < o[y].stride; });
  stat.insert(stat.end(), dyn.begin(), dyn.end());
  const std::vector<int64_t> strides = compact_in_order(m, stat);
  size_t at = 0;
  return map_leaves(shape, strides, at);
}

Layout logical_product(const Layout& block, const Layout& rest) {
  const Layout comp = complement(block, mul(size(block), cosize(rest)));
  return Layout::tuple({block, composition(comp, rest)});
}

Layout tiled_product(const Layout& block, const Layout& rest) {
  const Layout prod = logical_product(block, rest);
  std::vector<Layout> k{block};
  const Layout& r = prod.kids[1];
  for (size_t i = 0; i < r.rank(); ++i) k.push_back(r.at(i));
  return Layout::tuple(std::move(k));
}

Layout fragment_like(const Layout& partition) {
  const Layout& atom = partition.at(0);
  const Layout compact = compact_left(filter_zeros(atom));
  // the atom's own shape with the compact strides (broadcast leaves keep
  // their size and stride 0)
  std::vector<int64_t> strides;
  for (const Mode& x : flatten(compact)) strides.push_back(x.stride);
  size_t at = 0;
  const Layout block = map_leaves(atom, strides, at);
  if (partition.rank() < 2) return partition.leaf ? block : Layout::tuple({block});
  const Layout rest_modes = tuple_of_modes(partition, 1);
  const Layout rest = make_ordered(rest_modes, rest_modes);
  return tiled_product(block, rest);
}

Layout tensor_like(const Layout& partition) { return make_ordered(partition, partition); }

}  // namespace la
}  // namespace sl
