// kernels.hpp -- argument blocks and launchers of the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <cstdint>

#include "layout.hpp"

namespace lkv {

struct AppendArgs {
  uint8_t* pool;
  uint16_t* staging;            // [slots][H][32][D] bf16
  const int32_t* seq_lens;      // length before the append
  const int32_t* slots;         // may be null
  const int32_t* block_tables;
  const uint16_t* k_in;         // [B][n_new][H][D] bf16
  const uint16_t* v_in;
  int64_t num_pages;
  int32_t H, max_pages, n_new;
  CellLayout lay;
};

// Maximum split length whose scores fit the split kernel's LDS buffer.
constexpr int kMaxSplitLen = 4096;
// Maximum number of splits per (sequence, head).
constexpr int kMaxSplits = 2048;
constexpr int kTile = 64;            // tokens per wave iteration
constexpr int kPartialPad = 4;       // floats before o[] in a partial record

struct DecodeArgs {
  const uint8_t* pool;
  const int32_t* seq_lens;
  const int32_t* block_tables;
  const uint16_t* q;                 // [B][H][D] bf16
  float* out;                        // [B][H][D]
  float* partials;                   // [B][H][S][D + kPartialPad]
  int2* cand;                        // [B][H][S][split_len] (token, score bits)
  int32_t* cand_count;               // [B][H][S]
  uint32_t* mask_bits;               // optional [B][H][mask_words]
  unsigned long long* counters;      // optional [2]
  int64_t num_pages;
  int32_t H, max_pages, S, split_len, mask_words;
  int32_t grade_simds;               // one round of waves: the chip's SIMD count (block b is
                                     //    dispatched as wave b / grade_simds of its SIMD);
                                     //    0: several rounds, no issue-priority grading
  int32_t direct_out;                // 1: one uniform split per pair; a plain or dense
                                     //    split writes out itself, no merge launch
  float sm_scale;
  float log_tau;                     // ln(tau) for the candidate / flag test
  CellLayout lay;
  // Split layout.  Uniform (streamed == 0): the grid is (S, H, B) and split
  // k of a (sequence, head) covers tokens [k * split_len, (k + 1) *
  // split_len).  Streamed: the (sequence, head) pairs' 64-token tiles are
  // laid end to end (sequence-major, then head) and cut into consecutive
  // ranges: tiles_per_wave tiles for ranges below main_waves, tail_tiles
  // after.  Wave w of the 1-D grid (waves waves) takes range w, the last
  // wave also the ranges past the grid; each pair gets one partial record
  // per range that meets it.  S: partial records per pair; cand_stride:
  // candidate entries per pair (a record's list starts at its first token's
  // offset), also the cap on a length.
  int32_t streamed;
  int32_t tiles_per_wave;
  int32_t main_waves, tail_tiles;
  int32_t waves;                     // streamed: the grid
  int32_t batch;
  int32_t cand_stride;
};

// Sequences of a streamed layout (each wave scans all their lengths).
constexpr int kMaxStreamedBatch = 256;

// mode of a decode launch
enum DecodeMode : int {
  kModePlain = 0,      // 2-bit source, or 4-bit with tau = +inf: no low plane
  kModeSparse = 1,     // 4-bit, 0 < tau < inf: candidates + flagged gather
  kModeDense = 2,      // 4-bit, tau = 0: every low plane read in the split pass
};

// Measurement hook.  While profiling is enabled, prof_events(cls) hands out
// a fresh event pair for one launch of kernel class `cls`; the launch passes
// it to hipExtLaunchKernel, which stamps the kernel's own start and end on
// the launch stream (nothing is recorded between launches, so the timed
// kernels run back to back as they do unprofiled).  Otherwise both are null.
enum { kClassSplit = 0, kClassMerge = 1, kClassAppend = 2, kClasses = 3 };
struct ProfEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
ProfEvents prof_events(int cls);

hipError_t launch_append(const AppendArgs& a, int batch, hipStream_t stream);
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                             hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int batch, int mode, hipStream_t stream);
// log-sum-exp merge of plain partials only (no tau mask)
hipError_t launch_merge_plain(const DecodeArgs& a, int batch, hipStream_t stream);

// ---- joint vector quantization across loop steps (LoopVQ-style) ---------
constexpr int kVqSub = 4;            // channels per loop in one joint vector
constexpr int kVqCodes = 256;        // codewords per codebook (8-bit index)
constexpr int kVqSplitUnit = 512;   // decode split lengths are multiples of this (8 waves x 64 tokens)
constexpr int kVqSplitMax = 32768;   // tokens per decode split

struct VqArgs {
  uint8_t* pool;                     // [H][num_pages]: [P][D/4] key, then [P][D/4] value indices
  const uint16_t* cb_k;              // [R][256][D/4][4] fp16 codebook of the keys (loop-major)
  const uint16_t* cb_v;              // same for the values
  const int32_t* seq_lens;
  const int32_t* block_tables;
  const uint16_t* k_in;              // encode: [R][B][n_new][H][D] bf16
  const uint16_t* v_in;
  const uint16_t* q;                 // decode: [B][H][D] bf16
  float* partials;                   // decode: [B][H][S][D + kPartialPad]
  float* out;                        // decode: [B][H][D], written by the split pass when S == 1
  int64_t num_pages;
  int32_t R, batch, H, P, max_pages, n_new, loop, S, split_len;
  float sm_scale;
};

hipError_t launch_vq_encode(const VqArgs& a, int D, hipStream_t stream);
hipError_t launch_vq_split(const VqArgs& a, int D, hipStream_t stream);

}  // namespace lkv
