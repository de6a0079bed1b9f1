// layout_algebra.hpp -- host-side algebra of shape:stride layouts, the
// notation of "数据布局及其记号" (section "Shape-Stride 模型": a layout maps a
// coordinate to an offset by the dot product with the strides) and the
// operations "CuTe 中 A、B 如何加载到 MMA 寄存器" builds its fragments with
// (sections 2-3 and the closing source notes: composition of a tile with a
// TV slice, the inverse of a TV layout, division of a tensor by a tile,
// dropping broadcast modes, compact strides in a chosen order, and the
// product that places an atom's fragment under its repeats).
//
// Layouts are trees: a leaf is one (shape, stride) mode, an inner node a
// tuple of sub-layouts.  Coordinates are unflattened first-mode-fastest
// (colex), the convention the fragment page uses.  Strides are >= 0.
//
// Static and dynamic integers.  The fragment page separates values fixed at
// compile time (printed with a leading '_', e.g. "_8") from run-time ones
// (printed bare): only a static zero stride marks a broadcast mode for
// filter_zeros, and make_ordered puts modes with static order values first
// (by value) and those with run-time order values after them, in the order
// they appear.  parse() follows that printing convention: "_8" is static,
// "8" is run-time.  Layouts built in code (Layout::mode) are static, as the
// tile layouts of the kernels are compile-time constants.  Results carry a
// leaf static when everything it was computed from is static; compact
// strides made by compact_left / make_ordered are static.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

namespace sl {
namespace la {

struct Layout {
  bool leaf = true;
  int64_t shape = 1, stride = 0;   // leaf
  bool shape_static = true, stride_static = true;
  std::vector<Layout> kids;        // tuple

  static Layout mode(int64_t s, int64_t d, bool stat = true) {
    Layout l;
    l.shape = s;
    l.stride = d;
    l.shape_static = l.stride_static = stat;
    return l;
  }
  static Layout tuple(std::vector<Layout> k) {
    Layout l;
    l.leaf = false;
    l.kids = std::move(k);
    return l;
  }
  // top-level modes (a leaf is its own single mode)
  size_t rank() const { return leaf ? 1 : kids.size(); }
  const Layout& at(size_t i) const { return leaf ? *this : kids[i]; }
};

struct Mode {
  int64_t shape, stride;
  bool stat;  // stride static
};

// Thrown (as a message) when an operation is not defined for its operands.
struct Error {
  std::string what;
};

// "(4,(2,2)):(1,(4,8))", "8:1", "((_2,_2),_4):((_1,72),_2048)" -> Layout
Layout parse(const std::string& text);
// a shape tuple alone, "(2,(2,2))" (strides left static 0)
Layout parse_shape(const std::string& text);
// "(4,(2,2)):(1,(4,8))"; with mark_static, static values get a leading '_'
std::string to_string(const Layout& l, bool mark_static = false);

std::vector<Mode> flatten(const Layout& l);
int64_t size(const Layout& l);
int64_t cosize(const Layout& l);  // 1 + largest offset (0 for an empty layout)
int64_t eval(const Layout& l, int64_t index);
bool all_static(const Layout& l);

// size-1 modes dropped, adjacent modes with d1 == s0*d0 merged (flat result)
Layout coalesce(const Layout& l);
// A o B: B's hierarchy, each leaf of B composed with coalesce(A); A's last
// mode extends past its size.  Defined when every stride of B divides
// through A's shapes (or they divide it) and each B shape likewise.
Layout composition(const Layout& a, const Layout& b);
// the layout of increasing strides that fills [0, cosize_target) around
// A's image (A's strides nested multiples)
Layout complement(const Layout& a, int64_t cosize_target);
// R with A(R(i)) == i for i < size(R): the inverse on the contiguous prefix
// [0, size(R)) of A's image
Layout right_inverse(const Layout& a);
// ((tile modes), (rest modes)): each mode i of A divided by mode i of the
// tiler (a layout over that mode), the tile and rest parts zipped
Layout zipped_divide(const Layout& a, const Layout& tiler);
// the leaves of a whose stride is a static 0 get shape 1 (strides kept)
Layout filter_zeros(const Layout& a);
// compact first-mode-fastest strides for a's shape; size-1 modes get
// stride 0 and do not advance the running product
Layout compact_left(const Layout& a);
// compact strides for `shape`, assigned in the order of `order`'s leaves:
// static values ascending first, then run-time ones as they appear; size-1
// modes get stride 0
Layout make_ordered(const Layout& shape, const Layout& order);
// (block, complement(block, size(block)*cosize(rest)) o rest)
Layout logical_product(const Layout& block, const Layout& rest);
// the same with rest's top-level modes lifted next to block:
// (block, rest_0, rest_1, ...)
Layout tiled_product(const Layout& block, const Layout& rest);
// storage layout for a thread's values, from the thread's partition of a
// tile (mode 0: one instruction's values; modes 1..: its repeats):
//   block = (shape_0 : compact_left(filter_zeros(mode 0)))
//   rest  = make_ordered(shape of modes 1.., strides of modes 1..)
//   result = tiled_product(block, rest)
Layout fragment_like(const Layout& partition);
// make_ordered over all modes at once (the contrast the fragment page draws)
Layout tensor_like(const Layout& partition);

}  // namespace la
}  // namespace sl
