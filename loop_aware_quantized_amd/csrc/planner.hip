// planner.hip -- offline plan search: the storage kind of every (loop,
// layer) cell that minimizes decode reads under budgets for predicted
// damage and storage.
//
// Source: "LoopKV: Loop-Aware KV Cache Compression for Serving Looped
// Transformers", abstract (概要): the model's output damage is close to the
// sum of per-cell damages; a profile taken once, offline, selects per cell
// 4-bit codes, 2-bit codes or borrowing the last loop's cache, and the plan
// reads the fewest bytes while its predicted damage and storage stay within
// given limits.
//
// Host code only.  Exact search: the cells of one layer interact only
// through reuse (a loop that reuses reads the final loop's cell in that
// cell's format), so each layer has 2 * 3^(R-1) kind combinations.  A
// dynamic program over the layers keeps, for every (storage, reads) total,
// the least damage reached; reads and storage are whole multiples of 32
// bytes per token-head, so the state space is small and the result exact.
#include <cmath>
#include <cstdint>
#include <limits>
#include <new>
#include <vector>

#include "loopkv.h"

namespace lkv {
void set_last_error(const char* msg);
}

namespace {

// 32-byte units per token-head (D = 128: a 2-bit plane row is 32 B, the
// key + value metadata of a token-head 32 B)
constexpr int kReadQ4 = 4;    // K hi + lo, V hi, metadata
constexpr int kReadQ2 = 3;    // K, V, metadata
constexpr int kStoreQ4 = 5;   // four planes + metadata
constexpr int kStoreQ2 = 3;   // two planes + metadata

struct Combo {
  int store, reads;
  double damage;
  uint32_t kinds;   // 2 bits per loop, loop 0 in the low bits
};

int fail(int code, const char* msg) {
  lkv::set_last_error(msg);
  return code;
}

}  // namespace

static int plan_optimize(int32_t R, int32_t L, const double* damage, double damage_budget,
                         int64_t storage_budget, uint8_t* kinds, double* totals) {
  if (R < 1 || R > 8 || L < 1 || L > 4096) return fail(LOOPKV_E_INVAL, "plan_optimize: need 1 <= R <= 8, 1 <= L <= 4096");
  if (!damage || !kinds) return fail(LOOPKV_E_INVAL, "plan_optimize: NULL damage or kinds");
  if (!(damage_budget >= 0.0) || storage_budget < 0)
    return fail(LOOPKV_E_INVAL, "plan_optimize: budgets must be >= 0 (and not NaN)");
  const int64_t cells = static_cast<int64_t>(R) * L;
  for (int64_t i = 0; i < cells * 4; ++i)
    if (!(damage[i] >= 0.0) || !std::isfinite(damage[i]))
      return fail(LOOPKV_E_INVAL, "plan_optimize: damages must be finite and >= 0");

  // kind combinations of one layer, as (storage, reads, damage) per layer
  const int n_combo = 2 * static_cast<int>(std::pow(3.0, R - 1) + 0.5);
  const int s_layer = kStoreQ4 * R, r_layer = kReadQ4 * R;
  const int S_max = s_layer * L, RD_max = r_layer * L;
  const double inf = std::numeric_limits<double>::infinity();

  // dp[s][rd]: least damage over the layers so far; choice[l][s][rd]: combo
  const int64_t states = static_cast<int64_t>(S_max + 1) * (RD_max + 1);
  if (states * L > (int64_t(1) << 28))
    return fail(LOOPKV_E_INVAL, "plan_optimize: instance too large (R*L grid)");
  std::vector<double> dp(states, inf), next(states, inf);
  std::vector<uint16_t> choice(static_cast<size_t>(L) * states, 0);
  dp[0] = 0.0;
  std::vector<Combo> combos(n_combo);
  int s_hi = 0, rd_hi = 0;   // reachable bounds so far
  for (int l = 0; l < L; ++l) {
    for (int c = 0; c < n_combo; ++c) {
      // combo c: final-loop format from bit 0, loops 0..R-2 in base 3
      const int fin = c & 1;                  // 0: 4-bit, 1: 2-bit
      int rest = c >> 1;
      Combo cb{0, 0, 0.0, 0u};
      const double* dfin = damage + ((static_cast<int64_t>(R - 1) * L + l) * 4);
      for (int r = 0; r < R - 1; ++r) {
        const int k = rest % 3;               // LOOPKV_CELL_Q4 / Q2 / REUSE
        rest /= 3;
        const double* d = damage + ((static_cast<int64_t>(r) * L + l) * 4);
        if (k == LOOPKV_CELL_Q4) {
          cb.store += kStoreQ4; cb.reads += kReadQ4; cb.damage += d[0];
        } else if (k == LOOPKV_CELL_Q2) {
          cb.store += kStoreQ2; cb.reads += kReadQ2; cb.damage += d[1];
        } else {
          cb.reads += fin ? kReadQ2 : kReadQ4; cb.damage += fin ? d[3] : d[2];
        }
        cb.kinds |= static_cast<uint32_t>(k) << (2 * r);
      }
      cb.store += fin ? kStoreQ2 : kStoreQ4;
      cb.reads += fin ? kReadQ2 : kReadQ4;
      cb.damage += fin ? dfin[1] : dfin[0];
      cb.kinds |= static_cast<uint32_t>(fin ? LOOPKV_CELL_Q2 : LOOPKV_CELL_Q4) << (2 * (R - 1));
      combos[c] = cb;
    }
    // per (storage, reads) step keep the least-damage combination (the
    // first one on ties)
    std::vector<int> use;
    for (int c = 0; c < n_combo; ++c) {
      size_t i = 0;
      while (i < use.size() && (combos[use[i]].store != combos[c].store || combos[use[i]].reads != combos[c].reads)) ++i;
      if (i == use.size()) use.push_back(c);
      else if (combos[c].damage < combos[use[i]].damage) use[i] = c;
    }
    std::fill(next.begin(), next.end(), inf);
    uint16_t* ch = choice.data() + static_cast<size_t>(l) * states;
    for (int s = 0; s <= s_hi; ++s) {
      for (int rd = 0; rd <= rd_hi; ++rd) {
        const double base = dp[static_cast<int64_t>(s) * (RD_max + 1) + rd];
        if (base == inf) continue;
        for (int c : use) {
          const Combo& cb = combos[c];
          const int64_t idx = static_cast<int64_t>(s + cb.store) * (RD_max + 1) + rd + cb.reads;
          const double v = base + cb.damage;
          if (v < next[idx]) {
            next[idx] = v;
            ch[idx] = static_cast<uint16_t>(c);
          }
        }
      }
    }
    dp.swap(next);
    s_hi += s_layer;
    rd_hi += r_layer;
  }

  // least reads; then least damage; then least storage
  int best_s = -1, best_rd = -1;
  double best_d = inf;
  for (int rd = 0; rd <= RD_max && best_s < 0; ++rd) {
    for (int s = 0; s <= S_max && s <= storage_budget; ++s) {
      const double v = dp[static_cast<int64_t>(s) * (RD_max + 1) + rd];
      if (v <= damage_budget && v < best_d) {
        best_d = v;
        best_s = s;
        best_rd = rd;
      }
    }
  }
  if (best_s < 0) return fail(LOOPKV_E_PLAN, "plan_optimize: no plan meets both budgets");

  // walk the choices back, last layer first
  int s = best_s, rd = best_rd;
  for (int l = L - 1; l >= 0; --l) {
    const int64_t idx = static_cast<int64_t>(s) * (RD_max + 1) + rd;
    const int c = choice[static_cast<size_t>(l) * states + idx];
    // recompute the combo's totals (the table above was per layer)
    const int fin = c & 1;
    int rest = c >> 1;
    int cs = fin ? kStoreQ2 : kStoreQ4, cr = fin ? kReadQ2 : kReadQ4;
    for (int r = 0; r < R - 1; ++r) {
      const int k = rest % 3;
      rest /= 3;
      kinds[static_cast<int64_t>(r) * L + l] = static_cast<uint8_t>(k);
      if (k == LOOPKV_CELL_Q4) { cs += kStoreQ4; cr += kReadQ4; }
      else if (k == LOOPKV_CELL_Q2) { cs += kStoreQ2; cr += kReadQ2; }
      else cr += fin ? kReadQ2 : kReadQ4;
    }
    kinds[static_cast<int64_t>(R - 1) * L + l] = static_cast<uint8_t>(fin ? LOOPKV_CELL_Q2 : LOOPKV_CELL_Q4);
    s -= cs;
    rd -= cr;
  }
  if (totals) {
    totals[0] = best_rd;
    totals[1] = best_s;
    totals[2] = best_d;
  }
  return LOOPKV_OK;
}

// The search tables can take up to about 0.5 GiB of host memory: an
// allocation failure is reported as an error, not thrown across the ABI.
extern "C" int loopkv_plan_optimize(int32_t R, int32_t L, const double* damage, double damage_budget,
                                    int64_t storage_budget, uint8_t* kinds, double* totals) {
  try {
    return plan_optimize(R, L, damage, damage_budget, storage_budget, kinds, totals);
  } catch (const std::bad_alloc&) {
    return fail(LOOPKV_E_INVAL, "plan_optimize: out of host memory for the search tables");
  }
}
