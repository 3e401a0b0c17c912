// abi.hip -- host side of the C ABI declared in include/loopkv.h: plan
// parsing and validation, argument checks, split selection and launches.
//
// Source of the plan semantics: "LoopKV: Loop-Aware KV Cache Compression for
// Serving Looped Transformers", abstract (概要) -- a choice made ahead of
// time for every (loop, layer) cell between 4-bit codes, 2-bit codes and
// borrowing the last loop's cache of the layer; at decode the lower bits of
// a 4-bit value are loaded only for tokens whose weight under the cell's
// own query passes the cell's threshold tau.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "layout.hpp"
#include "loopkv.h"

struct loopkv_plan {
  int32_t R, L, H, D, G, P;
  std::vector<uint8_t> kind;   // [R*L]
  std::vector<float> tau;      // [R*L]
};

namespace {
thread_local std::string g_err;
}  // namespace

namespace lkv {
void set_last_error(const char* msg) { g_err = msg; }
}  // namespace lkv

namespace {

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int fail_hip(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return LOOPKV_E_HIP;
}

// LOOPKV_LOG=1: one line per append / decode call on stderr.
bool log_enabled() {
  const char* v = std::getenv("LOOPKV_LOG");
  return v && v[0] == '1' && v[1] == '\0';
}

const char* mode_name(int mode) {
  return mode == lkv::kModeSparse ? "sparse-tau" : mode == lkv::kModeDense ? "dense(tau=0)" : "plain";
}

// LOOPKV_DEBUG=1: validate device-resident lengths, page tables and slots
// on the host before a launch (read on every call, so it can be switched
// within a process).
bool debug_enabled() {
  const char* v = std::getenv("LOOPKV_DEBUG");
  return v && v[0] == '1' && v[1] == '\0';
}

int32_t rd_i32(const uint8_t* p) {
  int32_t v;
  std::memcpy(&v, p, 4);
  return v;
}

bool cell_ok(const loopkv_plan* plan, int loop, int layer) {
  return plan && loop >= 0 && loop < plan->R && layer >= 0 && layer < plan->L;
}

int cu_count() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= static_cast<int>(cache.size())) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

bool misaligned(const void* p, uintptr_t align) { return (reinterpret_cast<uintptr_t>(p) & (align - 1)) != 0; }

// sequences per call: the launch grids carry the batch in a dimension of at
// most 65535 blocks
constexpr int32_t kMaxBatch = 65535;

// Host-checkable properties of a batch descriptor that every call shares
// (NULL pointers and lengths are checked by the callers).
const char* batch_error(const loopkv_batch* b) {
  if (b->batch > kMaxBatch) return "batch must be <= 65535";
  if (misaligned(b->seq_lens, 4) || misaligned(b->slots, 4) || misaligned(b->block_tables, 4))
    return "seq_lens, slots and block_tables must be 4-byte aligned";
  return nullptr;
}

// Split layout of a decode.  Uniform: S splits of len tokens per (sequence,
// head).  Streamed: `waves` waves each take tpw tiles of the pairs' tiles
// laid end to end; S is the partial records a pair can have, len = tpw * 64
// the longest range.  cand_stride: candidate entries per pair.
struct Splits {
  int S, len;
  bool streamed = false;
  int tpw = 0, waves = 0, main_waves = 0, tail_tiles = 1;
  int64_t cand_stride = 0;
};

Splits uniform(int64_t tm, int64_t len) {
  Splits sp;
  sp.S = static_cast<int>((tm + len - 1) / len);
  sp.len = static_cast<int>(len);
  sp.cand_stride = static_cast<int64_t>(sp.S) * len;
  return sp;
}

// Split plan for `batch` sequences x `heads` of at most t_max tokens (sum
// of lengths t_sum when known, else 0).  One wave runs per non-empty split.
//  - near-uniform lengths: one round of resident waves (12 per CU), all
//    splits the same length;
//  - ragged lengths: about three rounds of non-empty splits, so that waves
//    that finish early pick up the remaining ones and the tail is short.
// Automatic splits hold at least 256 tokens (4 tiles), and long sequences
// over few pairs get longer splits so that no pair has more than
// kMaxSplits; a requested count gives splits of ceil(t_max / count) tokens
// rounded up to a tile.  No split exceeds kMaxSplitLen or the longest
// sequence rounded up to a tile.
// Streamed layout for a ragged batch.  The pairs' tiles are laid end to
// end; one round of waves (12 per compute unit) takes equal ranges of the
// first 90% of them, and a second round takes the rest in ranges of
// kTailTiles tiles.  Waves of the first round finish spread over ~25% of
// the launch (a SIMD issues its oldest wave first); the second round's
// waves start in the slots that free up first, so the short ranges fill the
// end of the launch instead of idle slots.  Short ranges also mean more
// records and more candidates (each record's running threshold sees fewer
// tokens) for the merge.  Measured on ragged-16k (64 x 16 pairs), whole
// decode step: 16-tile ranges 2.5-3% faster than one round of equal
// ranges; 8-tile ranges speed the split kernel 1% more but cost the merge
// 0.3 ms; 5% or 15% tails gain less.  Ranges hold at least 4 tiles and at
// most a split's 4096 tokens.  Needs the length sum, at most
// kMaxStreamedBatch sequences, and records per pair within the workspace's
// split capacity.
constexpr double kTailShare = 0.10;
constexpr int64_t kTailTiles = 16;

bool streamed_layout(int64_t batch, int64_t heads, int64_t tm, int64_t t_sum, int64_t slots, Splits* out) {
  if (t_sum <= 0 || batch > lkv::kMaxStreamedBatch) return false;
  const int64_t tiles_ub = heads * ((t_sum + lkv::kTile - 1) / lkv::kTile + batch);   // >= the real count
  // the kernels index tiles in 32 bits: bound the count by the lengths'
  // maximum too, since the sum is only a hint
  const int64_t tiles_max = heads * batch * ((tm + lkv::kTile - 1) / lkv::kTile);
  if (tiles_ub > (int64_t{1} << 30) || tiles_max > (int64_t{1} << 30)) return false;
  const int64_t main_tiles = static_cast<int64_t>(static_cast<double>(tiles_ub) * (1.0 - kTailShare));
  int64_t tpw = std::max<int64_t>(4, (main_tiles + slots - 1) / slots);
  tpw = std::min<int64_t>(tpw, lkv::kMaxSplitLen / lkv::kTile);
  const int64_t main_waves = std::min<int64_t>(slots, (tiles_ub + tpw - 1) / tpw);
  const int64_t tail_tiles = std::min<int64_t>(kTailTiles, tpw);
  const int64_t rest = std::max<int64_t>(0, tiles_ub - main_waves * tpw);
  const int64_t waves = main_waves + (rest + tail_tiles - 1) / tail_tiles;
  out->main_waves = static_cast<int>(main_waves);
  out->tail_tiles = static_cast<int>(tail_tiles);
  const int64_t pair_tiles = (tm + lkv::kTile - 1) / lkv::kTile;
  // A pair's n tiles meet at most ceil(n / tail) + 1 ranges (each range,
  // also past the grid, has tail_tiles or more), whatever the hint.
  const int64_t recs = (pair_tiles + tail_tiles - 1) / tail_tiles + 1;
  const int64_t s_cap = std::min<int64_t>(lkv::kMaxSplits, pair_tiles);
  if (recs > s_cap || waves > 0x7fffffff) return false;
  out->S = static_cast<int>(recs);
  out->len = static_cast<int>(tpw * lkv::kTile);
  out->streamed = true;
  out->tpw = static_cast<int>(tpw);
  out->waves = static_cast<int>(waves);
  out->cand_stride = round_up(tm, lkv::kTile);
  return true;
}

// stream_ok: the decode mode has a streamed kernel variant at one round of
// 12 waves per compute unit (the tau = 0 variant needs more registers)
Splits choose_splits(int64_t batch, int64_t heads, int t_max, int64_t t_sum, int requested,
                     bool stream_ok = true) {
  const int64_t tm = std::max<int64_t>(t_max, 1);
  const int64_t pairs = std::max<int64_t>(batch * heads, 1);
  const int64_t slots = static_cast<int64_t>(cu_count()) * 12;
  int64_t len;
  if (requested > 0) {
    len = round_up((tm + requested - 1) / requested, lkv::kTile);
    len = std::min<int64_t>(len, lkv::kMaxSplitLen);
    return uniform(tm, len);
  }
  const bool ragged = t_sum > 0 && t_sum * 100 < tm * batch * 85;
  Splits st;
  if (ragged && stream_ok && streamed_layout(batch, heads, tm, t_sum, slots, &st)) return st;
  if (ragged) {
    len = round_up((t_sum * heads + 3 * slots - 1) / (3 * slots), lkv::kTile);
  } else {
    const int64_t s0 = (slots + pairs - 1) / pairs;
    len = round_up((tm + s0 - 1) / s0, lkv::kTile);
  }
  len = std::max<int64_t>(len, std::min<int64_t>(256, round_up(tm, lkv::kTile)));
  // long sequences over few pairs: no more than kMaxSplits splits per pair
  len = std::max<int64_t>(len, round_up((tm + lkv::kMaxSplits - 1) / lkv::kMaxSplits, lkv::kTile));
  // no split longer than the longest sequence (the ragged rule asks for more
  // when pairs are many and short); the workspace's per-pair candidate
  // stride relies on it
  len = std::min<int64_t>(len, round_up(tm, lkv::kTile));
  len = std::min<int64_t>(len, lkv::kMaxSplitLen);
  return uniform(tm, len);
}

struct WorkspacePlan {
  size_t partials, counts, cand, total;
};

WorkspacePlan workspace_plan(int64_t batch, int64_t H, int64_t D, int64_t t_max) {
  const int64_t tm = std::max<int64_t>(t_max, 1);
  const int64_t s_cap = std::min<int64_t>(lkv::kMaxSplits, round_up(tm, lkv::kTile) / lkv::kTile);
  const int64_t cand_per_pair = round_up(tm, lkv::kTile) + std::min<int64_t>(lkv::kMaxSplitLen, round_up(tm, lkv::kTile));
  WorkspacePlan w;
  w.partials = static_cast<size_t>(round_up(batch * H * s_cap * (D + lkv::kPartialPad) * 4, 256));
  w.counts = static_cast<size_t>(round_up(batch * H * s_cap * 4, 256));
  w.cand = static_cast<size_t>(round_up(batch * H * cand_per_pair * 8, 256));
  w.total = w.partials + w.counts + w.cand;
  return w;
}

// LOOPKV_DEBUG=1: copy lengths / tables / slots to the host and check them.
int debug_check(const loopkv_batch* bt, int P, int64_t num_pages, int extra, int max_slots,
                hipStream_t stream) {
  const int B = bt->batch;
  std::vector<int32_t> lens(B), table(static_cast<size_t>(B) * bt->max_pages), slots;
  hipError_t e = hipMemcpyAsync(lens.data(), bt->seq_lens, B * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(table.data(), bt->block_tables, table.size() * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess && bt->slots && max_slots > 0) {
    slots.resize(B);
    e = hipMemcpyAsync(slots.data(), bt->slots, B * 4, hipMemcpyDeviceToHost, stream);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail_hip(e, "debug copy of batch metadata");
  for (int b = 0; b < B; ++b) {
    const int64_t T = static_cast<int64_t>(lens[b]) + extra;
    if (lens[b] < 0 || T > bt->max_seq_len)
      return fail(LOOPKV_E_INVAL, "seq_lens[" + std::to_string(b) + "] out of range");
    const int64_t pages = (T + P - 1) / P;
    for (int64_t p = 0; p < pages; ++p) {
      const int32_t v = table[static_cast<size_t>(b) * bt->max_pages + p];
      if (v < 0 || v >= num_pages)
        return fail(LOOPKV_E_INVAL, "block_tables[" + std::to_string(b) + "][" + std::to_string(p) +
                                        "] out of range");
    }
    if (!slots.empty() && (slots[b] < 0 || slots[b] >= max_slots))
      return fail(LOOPKV_E_INVAL, "slots[" + std::to_string(b) + "] out of range");
  }
  return LOOPKV_OK;
}

// ---- measurement hook: kernel-stamped event pairs, per kernel class -----
struct ProfClass {
  std::vector<hipEvent_t> ev;  // start, stop, start, stop, ...
  size_t used = 0;             // events handed out since the last collect
};

struct Profiler {
  std::mutex mu;
  bool on = false;
  ProfClass cls[lkv::kClasses];
};

Profiler& profiler() {
  static Profiler p;
  return p;
}

}  // namespace

namespace lkv {

ProfEvents prof_events(int c) {
  Profiler& p = profiler();
  std::lock_guard<std::mutex> lock(p.mu);
  ProfEvents out;
  if (!p.on) return out;
  ProfClass& pc = p.cls[c];
  while (pc.ev.size() < pc.used + 2) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return out;
    pc.ev.push_back(e);
  }
  out.start = pc.ev[pc.used];
  out.stop = pc.ev[pc.used + 1];
  pc.used += 2;
  return out;
}

}  // namespace lkv

extern "C" {

int loopkv_profile_enable(int on) {
  Profiler& p = profiler();
  std::lock_guard<std::mutex> lock(p.mu);
  p.on = on != 0;
  return LOOPKV_OK;
}

int loopkv_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || bytes < 16 || (reinterpret_cast<uintptr_t>(buf) & 15u))
    return fail(LOOPKV_E_INVAL, "read_probe: buffer must be 16-byte aligned and >= 16 bytes");
  const hipError_t e = lkv::launch_read_probe(buf, bytes, sink, cu_count() * 12,
                                              static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "read_probe: kernel launch");
  g_err.clear();
  return LOOPKV_OK;
}

int loopkv_profile_collect(int kernel_class, int64_t* launches, double* total_ms) {
  if (kernel_class < 0 || kernel_class >= lkv::kClasses || !launches || !total_ms)
    return fail(LOOPKV_E_INVAL, "profile_collect: bad kernel class or NULL output");
  Profiler& p = profiler();
  std::lock_guard<std::mutex> lock(p.mu);
  ProfClass& pc = p.cls[kernel_class];
  const size_t pairs = pc.used / 2;
  double ms = 0.0;
  for (size_t i = 0; i < pairs; ++i) {
    hipError_t e = hipEventSynchronize(pc.ev[2 * i + 1]);
    float t = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, pc.ev[2 * i], pc.ev[2 * i + 1]);
    if (e != hipSuccess) {
      pc.used = 0;
      return fail_hip(e, "profile_collect");
    }
    ms += t;
  }
  pc.used = 0;
  *launches = static_cast<int64_t>(pairs);
  *total_ms = ms;
  return LOOPKV_OK;
}

int loopkv_abi_version(void) { return LOOPKV_ABI_VERSION; }

const char* loopkv_last_error(void) { return g_err.c_str(); }

int loopkv_plan_load(const void* blob, size_t nbytes, loopkv_plan** out) {
  if (!out) return fail(LOOPKV_E_INVAL, "plan_load: out is NULL");
  *out = nullptr;
  if (!blob) return fail(LOOPKV_E_INVAL, "plan_load: blob is NULL");
  const uint8_t* p = static_cast<const uint8_t*>(blob);
  if (nbytes < 32) return fail(LOOPKV_E_PLAN, "plan_load: blob shorter than its 32-byte header");
  if (std::memcmp(p, "LKVP", 4) != 0) return fail(LOOPKV_E_PLAN, "plan_load: bad magic (want LKVP)");
  uint32_t version;
  std::memcpy(&version, p + 4, 4);
  if (version != 1) return fail(LOOPKV_E_PLAN, "plan_load: unsupported version " + std::to_string(version));
  const int32_t R = rd_i32(p + 8), L = rd_i32(p + 12), H = rd_i32(p + 16), D = rd_i32(p + 20),
                G = rd_i32(p + 24), P = rd_i32(p + 28);
  if (R < 1 || R > 4096 || L < 1 || L > 4096)
    return fail(LOOPKV_E_PLAN, "plan_load: loops and layers must be in [1, 4096]");
  if (H < 1 || H > 1024) return fail(LOOPKV_E_PLAN, "plan_load: heads must be in [1, 1024]");
  if (D != 64 && D != 128) return fail(LOOPKV_E_PLAN, "plan_load: head_dim must be 64 or 128");
  if (G != lkv::kGroup) return fail(LOOPKV_E_PLAN, "plan_load: group size must be 32");
  if (P != 16 && P != 32 && P != 64) return fail(LOOPKV_E_PLAN, "plan_load: page size must be 16, 32 or 64");
  const size_t cells = static_cast<size_t>(R) * L;
  if (nbytes != 32 + 8 * cells)
    return fail(LOOPKV_E_PLAN, "plan_load: blob size " + std::to_string(nbytes) + " != 32 + 8*R*L = " +
                                   std::to_string(32 + 8 * cells));
  loopkv_plan* plan = new (std::nothrow) loopkv_plan;
  if (!plan) return fail(LOOPKV_E_PLAN, "plan_load: out of host memory");
  plan->R = R; plan->L = L; plan->H = H; plan->D = D; plan->G = G; plan->P = P;
  try {
    plan->kind.resize(cells);
    plan->tau.resize(cells);
  } catch (const std::bad_alloc&) {
    delete plan;
    return fail(LOOPKV_E_PLAN, "plan_load: out of host memory");
  }
  for (size_t c = 0; c < cells; ++c) {
    const uint8_t* rec = p + 32 + 8 * c;
    const int loop = static_cast<int>(c / L), layer = static_cast<int>(c % L);
    float tau;
    std::memcpy(&tau, rec + 4, 4);
    const std::string where = "cell (" + std::to_string(loop) + ", " + std::to_string(layer) + ")";
    if (rec[0] > lkv::kKindReuse) {
      delete plan;
      return fail(LOOPKV_E_PLAN, "plan_load: " + where + " has unknown kind " + std::to_string(rec[0]));
    }
    if (rec[0] == lkv::kKindReuse && loop == R - 1) {
      delete plan;
      return fail(LOOPKV_E_PLAN, "plan_load: " + where + " is in the final loop and cannot reuse it");
    }
    if (std::isnan(tau) || tau < 0.0f) {
      delete plan;
      return fail(LOOPKV_E_PLAN, "plan_load: " + where + " has tau that is NaN or negative");
    }
    plan->kind[c] = rec[0];
    plan->tau[c] = tau;
  }
  *out = plan;
  return LOOPKV_OK;
}

void loopkv_plan_free(loopkv_plan* plan) { delete plan; }

int loopkv_plan_dims(const loopkv_plan* plan, int32_t dims[6]) {
  if (!plan || !dims) return fail(LOOPKV_E_INVAL, "plan_dims: NULL argument");
  dims[0] = plan->R; dims[1] = plan->L; dims[2] = plan->H;
  dims[3] = plan->D; dims[4] = plan->G; dims[5] = plan->P;
  return LOOPKV_OK;
}

int loopkv_cell_info(const loopkv_plan* plan, int loop, int layer, int* kind, float* tau, int* src_loop) {
  if (!cell_ok(plan, loop, layer)) return fail(LOOPKV_E_INVAL, "cell_info: no such cell");
  const size_t c = static_cast<size_t>(loop) * plan->L + layer;
  if (kind) *kind = plan->kind[c];
  if (tau) *tau = plan->tau[c];
  if (src_loop) *src_loop = plan->kind[c] == lkv::kKindReuse ? plan->R - 1 : loop;
  return LOOPKV_OK;
}

size_t loopkv_head_block_bytes(const loopkv_plan* plan, int loop, int layer) {
  if (!cell_ok(plan, loop, layer)) return 0;
  const int k = plan->kind[static_cast<size_t>(loop) * plan->L + layer];
  if (k == lkv::kKindReuse) return 0;
  return static_cast<size_t>(lkv::make_layout(k, plan->P, plan->D).HB);
}

size_t loopkv_pool_bytes(const loopkv_plan* plan, int loop, int layer, int64_t num_pages) {
  if (num_pages < 0) return 0;
  return loopkv_head_block_bytes(plan, loop, layer) * static_cast<size_t>(plan ? plan->H : 0) *
         static_cast<size_t>(num_pages);
}

size_t loopkv_staging_bytes(const loopkv_plan* plan, int loop, int layer, int32_t max_slots) {
  if (!cell_ok(plan, loop, layer) || max_slots < 0) return 0;
  if (plan->kind[static_cast<size_t>(loop) * plan->L + layer] == lkv::kKindReuse) return 0;
  return static_cast<size_t>(max_slots) * plan->H * lkv::kGroup * plan->D * 2;
}

size_t loopkv_decode_workspace_bytes(const loopkv_plan* plan, int32_t batch, int32_t max_seq_len) {
  if (!plan || batch < 0 || max_seq_len < 0) return 0;
  return workspace_plan(batch, plan->H, plan->D, max_seq_len).total;
}

int loopkv_decode_splits(const loopkv_plan* plan, int32_t batch, int32_t max_seq_len, int32_t sum_seq_lens,
                         int32_t num_splits, int32_t out[2]) {
  if (!plan || !out) return fail(LOOPKV_E_INVAL, "decode_splits: NULL plan or out");
  if (batch < 0 || max_seq_len < 0 || num_splits < 0)
    return fail(LOOPKV_E_INVAL, "decode_splits: negative batch, max_seq_len or num_splits");
  const Splits sp = choose_splits(batch, plan->H, max_seq_len, sum_seq_lens > 0 ? sum_seq_lens : 0, num_splits);
  if (sp.S > lkv::kMaxSplits) return fail(LOOPKV_E_INVAL, "decode_splits: max_seq_len needs too many splits");
  out[0] = sp.S;
  out[1] = sp.len;
  return LOOPKV_OK;
}

int loopkv_append(const loopkv_plan* plan, const loopkv_cell_mem* cells, int loop, int layer,
                  const loopkv_batch* batch, int32_t n_new, const void* k_bf16, const void* v_bf16,
                  void* stream) {
  if (!plan || !cells || !batch) return fail(LOOPKV_E_INVAL, "append: NULL plan, cells or batch");
  if (!cell_ok(plan, loop, layer)) return fail(LOOPKV_E_INVAL, "append: no such cell");
  const size_t c = static_cast<size_t>(loop) * plan->L + layer;
  if (plan->kind[c] == lkv::kKindReuse) {
    g_err.clear();
    return LOOPKV_NOOP_REUSE;
  }
  const loopkv_cell_mem& mem = cells[c];
  if (!mem.pool || !mem.staging) return fail(LOOPKV_E_INVAL, "append: cell pool or staging is NULL");
  if (mem.num_pages < 1) return fail(LOOPKV_E_INVAL, "append: cell has no pages");
  if (static_cast<uint64_t>(mem.num_pages) * lkv::make_layout(plan->kind[c], plan->P, plan->D).HB > 0xFFFFFFFFull)
    return fail(LOOPKV_E_INVAL, "append: one head's pool region (num_pages * head-block bytes) exceeds 4 GiB");
  if (batch->batch < 0) return fail(LOOPKV_E_INVAL, "append: negative batch");
  if (const char* be = batch_error(batch)) return fail(LOOPKV_E_INVAL, std::string("append: ") + be);
  if (n_new < 1) return fail(LOOPKV_E_INVAL, "append: n_new must be >= 1");
  if (batch->batch == 0) return LOOPKV_OK;
  if (!k_bf16 || !v_bf16) return fail(LOOPKV_E_INVAL, "append: NULL key or value input");
  if ((reinterpret_cast<uintptr_t>(k_bf16) | reinterpret_cast<uintptr_t>(v_bf16)) % 16 != 0)
    return fail(LOOPKV_E_INVAL, "append: key and value inputs must be 16-byte aligned");
  if (!batch->seq_lens || !batch->block_tables)
    return fail(LOOPKV_E_INVAL, "append: NULL seq_lens or block_tables");
  if (batch->max_pages < 1) return fail(LOOPKV_E_INVAL, "append: max_pages must be >= 1");
  if (static_cast<int64_t>(batch->max_pages) * plan->P < batch->max_seq_len)
    return fail(LOOPKV_E_INVAL, "append: max_pages * page_size < max_seq_len");
  if (batch->max_seq_len < n_new) return fail(LOOPKV_E_INVAL, "append: max_seq_len < n_new");
  if (!batch->slots && batch->batch > mem.max_slots)
    return fail(LOOPKV_E_CAPACITY, "append: batch exceeds the cell's staging slots");
  if (mem.max_slots < 1) return fail(LOOPKV_E_CAPACITY, "append: cell has no staging slots");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_enabled()) {
    const int rc = debug_check(batch, plan->P, mem.num_pages, n_new, mem.max_slots, s);
    if (rc != LOOPKV_OK) return rc;
  }
  lkv::AppendArgs a{};
  a.pool = static_cast<uint8_t*>(mem.pool);
  a.staging = static_cast<uint16_t*>(mem.staging);
  a.seq_lens = batch->seq_lens;
  a.slots = batch->slots;
  a.block_tables = batch->block_tables;
  a.k_in = static_cast<const uint16_t*>(k_bf16);
  a.v_in = static_cast<const uint16_t*>(v_bf16);
  a.num_pages = mem.num_pages;
  a.H = plan->H;
  a.max_pages = batch->max_pages;
  a.n_new = n_new;
  a.lay = lkv::make_layout(plan->kind[c], plan->P, plan->D);
  if (log_enabled())
    std::fprintf(stderr, "[loopkv] append cell (%d,%d) %s batch=%d n_new=%d max_seq_len=%d\n", loop, layer,
                 plan->kind[c] == lkv::kKindQ4 ? "4-bit" : "2-bit", batch->batch, n_new, batch->max_seq_len);
  const hipError_t e = lkv::launch_append(a, batch->batch, s);
  if (e != hipSuccess) return fail_hip(e, "append: kernel launch");
  g_err.clear();
  return LOOPKV_OK;
}

}  // extern "C"

// ---- decode: shared by the workspace and the allocation-free entry points --

namespace {

// File-scope scratch of the allocation-free decode: one copy per GPU, held
// until the process ends.  Host code never passes `scratch` itself to a
// kernel (on the host it is only a stand-in for the symbol); it uses the
// device address looked up once per device by static_scratch_ptr().
constexpr size_t kStaticScratchBytes = LOOPKV_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

// Device address of `scratch` on the current device (NULL on failure, with
// the HIP error in *err).  Looked up with that device current on its first
// use and kept per device.
uint8_t* static_scratch_ptr(hipError_t* err) {
  static std::mutex mu;
  static std::vector<uint8_t*> by_device;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= static_cast<int>(by_device.size())) by_device.resize(dev + 1, nullptr);
  if (!by_device[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    by_device[dev] = static_cast<uint8_t*>(ptr);
  }
  *err = hipSuccess;
  return by_device[dev];
}

// Scratch an allocation-free decode of this batch uses: partial records and
// candidate counts for the chosen split layout, and candidate lists (one
// entry per token of a split) only when a tau mask is formed.
struct CompactScratch {
  size_t partials, counts, cand, total;
};

CompactScratch compact_scratch(int64_t batch, int64_t H, int64_t D, const Splits& sp, bool sparse) {
  const int64_t recs = batch * H * sp.S;
  CompactScratch c;
  c.partials = static_cast<size_t>(round_up(recs * (D + lkv::kPartialPad) * 4, 256));
  c.counts = static_cast<size_t>(round_up(recs * 4, 256));
  c.cand = sparse ? static_cast<size_t>(round_up(batch * H * sp.cand_stride * 8, 256)) : 0;
  c.total = c.partials + c.counts + c.cand;
  return c;
}

int decode_mode(int src_kind, float tau) {
  if (src_kind != lkv::kKindQ4) return lkv::kModePlain;
  if (tau == 0.0f) return lkv::kModeDense;
  return std::isfinite(tau) ? lkv::kModeSparse : lkv::kModePlain;
}

// Everything loopkv_decode checks and launches.  static_scratch: take the
// partials and candidate lists from the file-scope scratch (sized by the
// actual split layout) instead of opts->workspace.
int decode_impl(const char* who, const loopkv_plan* plan, const loopkv_cell_mem* cells, int loop, int layer,
                const loopkv_batch* batch, const void* q_bf16, float* out, const loopkv_decode_opts* opts,
                void* stream, bool static_scratch) {
  const std::string w(who);
  if (!plan || !cells || !batch || !opts) return fail(LOOPKV_E_INVAL, w + ": NULL plan, cells, batch or opts");
  if (!cell_ok(plan, loop, layer)) return fail(LOOPKV_E_INVAL, w + ": no such cell");
  const size_t c = static_cast<size_t>(loop) * plan->L + layer;
  const int src_loop = plan->kind[c] == lkv::kKindReuse ? plan->R - 1 : loop;
  const size_t sc = static_cast<size_t>(src_loop) * plan->L + layer;
  const int src_kind = plan->kind[sc];
  const float tau = plan->tau[c];
  const loopkv_cell_mem& mem = cells[sc];
  if (!mem.pool) return fail(LOOPKV_E_INVAL, w + ": source cell pool is NULL");
  if (mem.num_pages < 1) return fail(LOOPKV_E_INVAL, w + ": source cell has no pages");
  if (static_cast<uint64_t>(mem.num_pages) * lkv::make_layout(src_kind, plan->P, plan->D).HB > 0xFFFFFFFFull)
    return fail(LOOPKV_E_INVAL, w + ": one head's pool region (num_pages * head-block bytes) exceeds 4 GiB");
  if (batch->batch < 0) return fail(LOOPKV_E_INVAL, w + ": negative batch");
  if (const char* be = batch_error(batch)) return fail(LOOPKV_E_INVAL, w + ": " + be);
  if (opts->num_splits < 0) return fail(LOOPKV_E_INVAL, w + ": num_splits must be >= 0");
  if (batch->max_seq_len < 0) return fail(LOOPKV_E_INVAL, w + ": negative max_seq_len");
  if (!std::isfinite(opts->sm_scale)) return fail(LOOPKV_E_INVAL, w + ": sm_scale must be finite");
  if (batch->batch == 0) return LOOPKV_OK;
  if (!q_bf16 || !out) return fail(LOOPKV_E_INVAL, w + ": NULL query or output");
  if (misaligned(q_bf16, 2) || misaligned(out, 4) || misaligned(opts->mask_bits, 4) ||
      misaligned(opts->counters, 8))
    return fail(LOOPKV_E_INVAL, w + ": q must be 2-byte, out and mask_bits 4-byte, counters 8-byte aligned");
  if (!batch->seq_lens || !batch->block_tables)
    return fail(LOOPKV_E_INVAL, w + ": NULL seq_lens or block_tables");
  if (batch->max_pages < 1) return fail(LOOPKV_E_INVAL, w + ": max_pages must be >= 1");
  if (static_cast<int64_t>(batch->max_pages) * plan->P < batch->max_seq_len)
    return fail(LOOPKV_E_INVAL, w + ": max_pages * page_size < max_seq_len");
  const int mode = decode_mode(src_kind, tau);
  const Splits sp = choose_splits(batch->batch, plan->H, batch->max_seq_len,
                                  batch->sum_seq_lens > 0 ? batch->sum_seq_lens : 0, opts->num_splits,
                                  mode != lkv::kModeDense);
  if (sp.S > lkv::kMaxSplits) return fail(LOOPKV_E_INVAL, w + ": max_seq_len needs too many splits");

  uint8_t* ws;
  size_t off_counts, off_cand;
  if (static_scratch) {
    const CompactScratch cs = compact_scratch(batch->batch, plan->H, plan->D, sp, mode == lkv::kModeSparse);
    if (cs.total > kStaticScratchBytes)
      return fail(LOOPKV_E_CAPACITY, w + ": this batch needs " + std::to_string(cs.total) +
                                         " bytes of scratch, above the library's fixed " +
                                         std::to_string(kStaticScratchBytes));
    hipError_t e = hipSuccess;
    ws = static_scratch_ptr(&e);
    if (!ws) return fail_hip(e, (w + ": device address of the static scratch").c_str());
    off_counts = cs.partials;
    off_cand = cs.partials + cs.counts;
  } else {
    const WorkspacePlan wp = workspace_plan(batch->batch, plan->H, plan->D, batch->max_seq_len);
    if (!opts->workspace || opts->workspace_bytes < wp.total)
      return fail(LOOPKV_E_CAPACITY, w + ": workspace smaller than loopkv_decode_workspace_bytes (" +
                                         std::to_string(wp.total) + " bytes)");
    ws = static_cast<uint8_t*>(opts->workspace);
    off_counts = wp.partials;
    off_cand = wp.partials + wp.counts;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_enabled()) {
    const int rc = debug_check(batch, plan->P, mem.num_pages, 0, 0, s);
    if (rc != LOOPKV_OK) return rc;
  }
  lkv::DecodeArgs a{};
  a.pool = static_cast<const uint8_t*>(mem.pool);
  a.seq_lens = batch->seq_lens;
  a.block_tables = batch->block_tables;
  a.q = static_cast<const uint16_t*>(q_bf16);
  a.out = out;
  a.partials = reinterpret_cast<float*>(ws);
  a.cand_count = reinterpret_cast<int32_t*>(ws + off_counts);
  a.cand = reinterpret_cast<int2*>(ws + off_cand);
  a.mask_bits = opts->mask_bits;
  a.counters = opts->counters;
  a.num_pages = mem.num_pages;
  a.H = plan->H;
  a.max_pages = batch->max_pages;
  a.S = sp.S;
  a.split_len = sp.len;
  a.streamed = sp.streamed ? 1 : 0;
  a.tiles_per_wave = sp.tpw;
  a.waves = sp.waves;
  a.main_waves = sp.main_waves;
  a.tail_tiles = sp.tail_tiles;
  a.batch = batch->batch;
  a.cand_stride = static_cast<int32_t>(sp.cand_stride);
  const int64_t waves = sp.streamed ? sp.waves : static_cast<int64_t>(sp.S) * plan->H * batch->batch;
  // one round of resident waves (3 per SIMD): issue priority is graded by progress and dispatch rank
  a.grade_simds = waves <= static_cast<int64_t>(cu_count()) * 12 ? cu_count() * 4 : 0;
  // one split per pair and no tau test: the split writes the output itself
  a.direct_out = (!sp.streamed && sp.S == 1 && mode != lkv::kModeSparse) ? 1 : 0;
  a.mask_words = (batch->max_seq_len + 31) / 32;
  a.sm_scale = opts->sm_scale;
  a.log_tau = (mode == lkv::kModeSparse) ? std::log(tau) : 0.0f;
  a.lay = lkv::make_layout(src_kind, plan->P, plan->D);
  if (log_enabled()) {
    // plan-required bytes of the split pass: per token-head D (4-bit source:
    // both key planes, high value plane, metadata) or 3D/4 (2-bit), plus the
    // low plane D/4 when tau = 0
    const int64_t per = (src_kind == lkv::kKindQ4 ? plan->D : 3 * plan->D / 4) +
                        (mode == lkv::kModeDense ? plan->D / 4 : 0);
    const bool hint = batch->sum_seq_lens > 0;
    const int64_t tokens = hint ? batch->sum_seq_lens : static_cast<int64_t>(batch->batch) * batch->max_seq_len;
    std::fprintf(stderr,
                 "[loopkv] %s cell (%d,%d) src (%d,%d) %s %s tau=%g batch=%d max_seq_len=%d splits=%d x %d "
                 "tokens, required split-pass bytes %s%lld\n",
                 who, loop, layer, src_loop, layer, src_kind == lkv::kKindQ4 ? "4-bit" : "2-bit", mode_name(mode),
                 static_cast<double>(tau), batch->batch, batch->max_seq_len, sp.S, sp.len, hint ? "" : "<= ",
                 static_cast<long long>(tokens * plan->H * per));
  }
  const hipError_t e = lkv::launch_decode(a, batch->batch, mode, s);
  if (e != hipSuccess) return fail_hip(e, (w + ": kernel launch").c_str());
  g_err.clear();
  return LOOPKV_OK;
}

}  // namespace

extern "C" {

int loopkv_decode(const loopkv_plan* plan, const loopkv_cell_mem* cells, int loop, int layer,
                  const loopkv_batch* batch, const void* q_bf16, float* out,
                  const loopkv_decode_opts* opts, void* stream) {
  return decode_impl("decode", plan, cells, loop, layer, batch, q_bf16, out, opts, stream, false);
}

int loopkv_decode_layout(const loopkv_plan* plan, int loop, int layer, int32_t batch, int32_t max_seq_len,
                         int32_t sum_seq_lens, int32_t num_splits, int32_t out[4]) {
  if (!cell_ok(plan, loop, layer) || !out) return fail(LOOPKV_E_INVAL, "decode_layout: bad cell or NULL out");
  if (batch < 0 || max_seq_len < 0 || num_splits < 0)
    return fail(LOOPKV_E_INVAL, "decode_layout: negative batch, max_seq_len or num_splits");
  const size_t c = static_cast<size_t>(loop) * plan->L + layer;
  const int src_loop = plan->kind[c] == lkv::kKindReuse ? plan->R - 1 : loop;
  const int src_kind = plan->kind[static_cast<size_t>(src_loop) * plan->L + layer];
  const Splits sp = choose_splits(batch, plan->H, max_seq_len, sum_seq_lens > 0 ? sum_seq_lens : 0, num_splits,
                                  decode_mode(src_kind, plan->tau[c]) != lkv::kModeDense);
  if (sp.S > lkv::kMaxSplits) return fail(LOOPKV_E_INVAL, "decode_layout: max_seq_len needs too many splits");
  out[0] = sp.streamed ? 1 : 0;
  out[1] = sp.S;
  out[2] = sp.len;
  out[3] = sp.streamed ? sp.waves : 0;
  return LOOPKV_OK;
}

size_t loopkv_decode_noalloc_bytes(const loopkv_plan* plan, int loop, int layer, int32_t batch,
                                   int32_t max_seq_len, int32_t sum_seq_lens, int32_t num_splits) {
  if (!cell_ok(plan, loop, layer) || batch < 0 || max_seq_len < 0 || num_splits < 0) return 0;
  const size_t c = static_cast<size_t>(loop) * plan->L + layer;
  const int src_loop = plan->kind[c] == lkv::kKindReuse ? plan->R - 1 : loop;
  const int src_kind = plan->kind[static_cast<size_t>(src_loop) * plan->L + layer];
  const int mode = decode_mode(src_kind, plan->tau[c]);
  const Splits sp = choose_splits(batch, plan->H, max_seq_len, sum_seq_lens > 0 ? sum_seq_lens : 0, num_splits,
                                  mode != lkv::kModeDense);
  return compact_scratch(batch, plan->H, plan->D, sp, mode == lkv::kModeSparse).total;
}

int loopkv_decode_noalloc(const loopkv_plan* plan, const loopkv_cell_mem* cells, int loop, int layer,
                          const loopkv_batch* batch, const void* q_bf16, float* out,
                          const loopkv_decode_opts* opts, void* stream) {
  return decode_impl("decode_noalloc", plan, cells, loop, layer, batch, q_bf16, out, opts, stream, true);
}

// ---- joint vector quantization across loop steps -------------------------

namespace {

const char* vq_dims_error(const loopkv_vq_dims* d) {
  if (!d) return "vq: NULL dims";
  if (d->loops < 2 || d->loops > 4) return "vq: loops must be 2, 3 or 4";
  if (d->heads < 1 || d->heads > 1024) return "vq: heads must be in [1, 1024]";
  if (d->head_dim != 64 && d->head_dim != 128) return "vq: head_dim must be 64 or 128";
  if (d->page != 16 && d->page != 32 && d->page != 64) return "vq: page must be 16, 32 or 64";
  return nullptr;
}

int64_t vq_head_block(const loopkv_vq_dims* d) {
  return static_cast<int64_t>(2) * d->page * (d->head_dim / lkv::kVqSub);
}

struct VqSplits {
  int S, len;
};

// One block of 8 waves per compute unit is resident (its tables fill most
// of the LDS) and every block first builds its tables: as few splits as
// fill the compute units once, each a whole number of 512-token units and
// at most kVqSplitMax tokens.
VqSplits vq_splits(int64_t batch, int64_t heads, int t_max) {
  const int64_t tm = std::max<int64_t>(t_max, 1);
  int64_t s0 = std::max<int64_t>(1, (static_cast<int64_t>(cu_count()) + batch * heads - 1) / (batch * heads));
  s0 = std::max<int64_t>(s0, (tm + lkv::kVqSplitMax - 1) / lkv::kVqSplitMax);
  const int64_t len = std::min<int64_t>(round_up((tm + s0 - 1) / s0, lkv::kVqSplitUnit), lkv::kVqSplitMax);
  return {static_cast<int>((tm + len - 1) / len), static_cast<int>(len)};
}

}  // namespace

size_t loopkv_vq_codebook_bytes(const loopkv_vq_dims* d) {
  if (vq_dims_error(d)) return 0;
  return static_cast<size_t>(d->head_dim / lkv::kVqSub) * lkv::kVqCodes * lkv::kVqSub * d->loops * 2;
}

size_t loopkv_vq_pool_bytes(const loopkv_vq_dims* d, int64_t num_pages) {
  if (vq_dims_error(d) || num_pages < 0) return 0;
  return static_cast<size_t>(d->heads) * num_pages * vq_head_block(d);
}

size_t loopkv_vq_workspace_bytes(const loopkv_vq_dims* d, int32_t batch, int32_t max_seq_len) {
  if (vq_dims_error(d) || batch < 0 || max_seq_len < 0) return 0;
  const int64_t s_max = (std::max<int64_t>(max_seq_len, 1) + lkv::kVqSplitUnit - 1) / lkv::kVqSplitUnit;
  return static_cast<size_t>(round_up(static_cast<int64_t>(batch) * d->heads * s_max * (d->head_dim + lkv::kPartialPad) * 4, 256));
}

int loopkv_vq_append(const loopkv_vq_dims* d, void* pool, int64_t num_pages, const void* codebook_k,
                     const void* codebook_v, const loopkv_batch* batch, int32_t n_new, const void* k_bf16,
                     const void* v_bf16, void* stream) {
  if (const char* e = vq_dims_error(d)) return fail(LOOPKV_E_INVAL, e);
  if (!pool || !codebook_k || !codebook_v || !batch || !k_bf16 || !v_bf16)
    return fail(LOOPKV_E_INVAL, "vq_append: NULL pointer");
  if (n_new < 1) return fail(LOOPKV_E_INVAL, "vq_append: n_new must be >= 1");
  if (num_pages < 1) return fail(LOOPKV_E_INVAL, "vq_append: num_pages must be >= 1");
  if (batch->batch < 0 || batch->max_pages < 1 || !batch->seq_lens || !batch->block_tables)
    return fail(LOOPKV_E_INVAL, "vq_append: bad batch");
  if (const char* be = batch_error(batch)) return fail(LOOPKV_E_INVAL, std::string("vq_append: ") + be);
  if (static_cast<int64_t>(batch->max_pages) * d->page < batch->max_seq_len)
    return fail(LOOPKV_E_INVAL, "vq_append: max_pages * page < max_seq_len");
  if ((reinterpret_cast<uintptr_t>(k_bf16) | reinterpret_cast<uintptr_t>(v_bf16) |
       reinterpret_cast<uintptr_t>(codebook_k) | reinterpret_cast<uintptr_t>(codebook_v)) % 8 != 0)
    return fail(LOOPKV_E_INVAL, "vq_append: inputs and codebooks must be 8-byte aligned");
  if (batch->batch == 0) return LOOPKV_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_enabled()) {
    const int rc = debug_check(batch, d->page, num_pages, n_new, 0, s);
    if (rc != LOOPKV_OK) return rc;
  }
  lkv::VqArgs a{};
  a.pool = static_cast<uint8_t*>(pool);
  a.cb_k = static_cast<const uint16_t*>(codebook_k);
  a.cb_v = static_cast<const uint16_t*>(codebook_v);
  a.seq_lens = batch->seq_lens;
  a.block_tables = batch->block_tables;
  a.k_in = static_cast<const uint16_t*>(k_bf16);
  a.v_in = static_cast<const uint16_t*>(v_bf16);
  a.num_pages = num_pages;
  a.R = d->loops;
  a.batch = batch->batch;
  a.H = d->heads;
  a.P = d->page;
  a.max_pages = batch->max_pages;
  a.n_new = n_new;
  const hipError_t e = lkv::launch_vq_encode(a, d->head_dim, s);
  if (e != hipSuccess) return fail_hip(e, "vq_append: kernel launch");
  g_err.clear();
  return LOOPKV_OK;
}

int loopkv_vq_decode(const loopkv_vq_dims* d, const void* pool, int64_t num_pages, const void* codebook_k,
                     const void* codebook_v, int loop, const loopkv_batch* batch, const void* q_bf16, float* out,
                     float sm_scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (const char* e = vq_dims_error(d)) return fail(LOOPKV_E_INVAL, e);
  if (loop < 0 || loop >= d->loops) return fail(LOOPKV_E_INVAL, "vq_decode: loop out of range");
  if (!pool || !codebook_k || !codebook_v || !batch || !q_bf16 || !out || !workspace)
    return fail(LOOPKV_E_INVAL, "vq_decode: NULL pointer");
  if (num_pages < 1) return fail(LOOPKV_E_INVAL, "vq_decode: num_pages must be >= 1");
  if (batch->batch < 0 || batch->max_pages < 1 || !batch->seq_lens || !batch->block_tables || batch->max_seq_len < 0)
    return fail(LOOPKV_E_INVAL, "vq_decode: bad batch");
  if (const char* be = batch_error(batch)) return fail(LOOPKV_E_INVAL, std::string("vq_decode: ") + be);
  if (misaligned(out, 4) || !std::isfinite(sm_scale))
    return fail(LOOPKV_E_INVAL, "vq_decode: out must be 4-byte aligned and sm_scale finite");
  if (static_cast<int64_t>(batch->max_pages) * d->page < batch->max_seq_len)
    return fail(LOOPKV_E_INVAL, "vq_decode: max_pages * page < max_seq_len");
  if (reinterpret_cast<uintptr_t>(q_bf16) % 8 != 0 ||
      (reinterpret_cast<uintptr_t>(codebook_k) | reinterpret_cast<uintptr_t>(codebook_v) |
       reinterpret_cast<uintptr_t>(pool)) % 16 != 0)
    return fail(LOOPKV_E_INVAL, "vq_decode: the query must be 8-byte, codebooks and pool 16-byte aligned");
  if (workspace_bytes < loopkv_vq_workspace_bytes(d, batch->batch, batch->max_seq_len))
    return fail(LOOPKV_E_CAPACITY, "vq_decode: workspace smaller than loopkv_vq_workspace_bytes");
  if (batch->batch == 0) return LOOPKV_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_enabled()) {
    const int rc = debug_check(batch, d->page, num_pages, 0, 0, s);
    if (rc != LOOPKV_OK) return rc;
  }
  const VqSplits sp = vq_splits(batch->batch, d->heads, batch->max_seq_len);
  lkv::VqArgs a{};
  a.pool = static_cast<uint8_t*>(const_cast<void*>(pool));
  a.cb_k = static_cast<const uint16_t*>(codebook_k);
  a.cb_v = static_cast<const uint16_t*>(codebook_v);
  a.seq_lens = batch->seq_lens;
  a.block_tables = batch->block_tables;
  a.q = static_cast<const uint16_t*>(q_bf16);
  a.partials = static_cast<float*>(workspace);
  a.num_pages = num_pages;
  a.R = d->loops;
  a.batch = batch->batch;
  a.H = d->heads;
  a.P = d->page;
  a.max_pages = batch->max_pages;
  a.loop = loop;
  a.S = sp.S;
  a.split_len = sp.len;
  a.sm_scale = sm_scale;
  a.out = out;
  hipError_t e = lkv::launch_vq_split(a, d->head_dim, s);
  if (e != hipSuccess) return fail_hip(e, "vq_decode: split kernel launch");
  if (sp.S == 1) {         // the split pass wrote the output
    g_err.clear();
    return LOOPKV_OK;
  }
  lkv::DecodeArgs m{};
  m.seq_lens = batch->seq_lens;
  m.block_tables = batch->block_tables;
  m.out = out;
  m.partials = static_cast<float*>(workspace);
  m.H = d->heads;
  m.max_pages = batch->max_pages;
  m.S = sp.S;
  m.split_len = sp.len;
  m.lay = lkv::make_layout(lkv::kKindQ2, d->page, d->head_dim);
  e = lkv::launch_merge_plain(m, batch->batch, s);
  if (e != hipSuccess) return fail_hip(e, "vq_decode: merge kernel launch");
  g_err.clear();
  return LOOPKV_OK;
}

}  // extern "C"
