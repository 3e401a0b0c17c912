// layout.hpp -- byte layout of one stored cell's paged pool.
//
// Source: "LoopKV: Loop-Aware KV Cache Compression for Serving Looped
// Transformers", abstract (概要): a cell keeps 4-bit or 2-bit codes, and
// the upper two bits of a 4-bit code are used without the lower two, so a
// 4-bit cell keeps separate high and low planes.  Keys are grouped per
// channel over 32 tokens and values per token over 32 channels (the KIVI
// entry of the related-papers list on the fugumt LoopVQ page).
//
// Head-block of head h, physical page p, at byte (h * num_pages + p) * HB:
//   4-bit: K_hi | K_lo | V_hi | V_lo | Vmeta | Kmeta
//   2-bit: K    | V    | Vmeta | Kmeta
// rows are token-major, D/4 bytes each; Vmeta is [P][D/32]{f16 s, f16 z};
// Kmeta has max(1, P/32) slots of {f16 scale[D], f16 zero[D]}.
#pragma once

#include <cstdint>

namespace lkv {

constexpr int kGroup = 32;
constexpr int kKindQ4 = 0;
constexpr int kKindQ2 = 1;
constexpr int kKindReuse = 2;

struct CellLayout {
  int32_t kind;      // kKindQ4 or kKindQ2
  int32_t P, D;      // page tokens, head dim
  int32_t row;       // bytes per row = D / 4
  int32_t off_khi;   // K (2-bit cell) or K high plane
  int32_t off_klo;   // K low plane (4-bit cell only, else -1)
  int32_t off_vhi;   // V (2-bit cell) or V high plane
  int32_t off_vlo;   // V low plane (4-bit cell only, else -1)
  int32_t off_vmeta;
  int32_t off_kmeta;
  int32_t kslots;
  int32_t HB;        // head-block bytes
};

inline CellLayout make_layout(int kind, int P, int D) {
  CellLayout L{};
  L.kind = kind;
  L.P = P;
  L.D = D;
  L.row = D / 4;
  const int plane = P * L.row;
  int off;
  if (kind == kKindQ4) {
    L.off_khi = 0;
    L.off_klo = plane;
    L.off_vhi = 2 * plane;
    L.off_vlo = 3 * plane;
    off = 4 * plane;
  } else {
    L.off_khi = 0;
    L.off_klo = -1;
    L.off_vhi = plane;
    L.off_vlo = -1;
    off = 2 * plane;
  }
  L.off_vmeta = off;
  off += P * (D / kGroup) * 4;
  L.kslots = P >= kGroup ? P / kGroup : 1;
  L.off_kmeta = off;
  off += L.kslots * D * 4;
  L.HB = off;
  return L;
}

}  // namespace lkv
