// vq.hip -- joint vector quantization of keys and values across loop steps,
// and the split pass of decode attention over such a cache (LoopVQ-style).
//
// Source: "LoopVQ: Sub 1-bit KV Cache Quantization for Looped
// Transformers", abstract (概要): keys and values change little from one
// loop step to the next, so one codebook entry can stand for a group of
// channels of all loop steps at once, at half a bit per element.
//
// Format: for one layer, token and head, channel group j's joint vector is
// the concatenation over loops r of channels [4j, 4j+4) of loop r's key (or
// value), 4R numbers; group j's codebook holds 256 codewords (fp16), so one
// byte codes 4R elements (R = 4: 0.5 bit per element).  All loops of a
// layer share one index cache; loop r decodes slice [4r, 4r+4) of each
// codeword.
//
// Codebook layout: [R][256][G][4] fp16 (G = D/4), loop r's 4 channels of
// codeword c of group j at ((r * 256 + c) * G + j) * 4, so a decode of one
// loop reads one contiguous slice.
//
// Layout of a head-block (one head, one page of P tokens): P key index
// rows of D/4 bytes, then P value index rows of D/4 bytes (token-major), so
// the 64 lanes of a wave read one 64-token tile's rows as contiguous runs.
// Group j of the token at position t is byte j ^ (t mod D/4) of its row.
//
// Decode of loop r, one block of 8 waves per (split, head, sequence):
//   1. a table of sm_scale * q[4j..4j+4) . key codeword_c[4r..4r+4) for
//      every group j and code c, and the loop's value codeword slices, both
//      in LDS, so a token's score is the sum of D/4 table reads addressed by
//      its key bytes;
//   2. each wave streams its own 64-token tiles (lane = token) with a
//      per-lane softmax reference: score, p_t, and per value group one LDS
//      read of the 4 fp16 channels of the chosen codeword and 4 FMAs into
//      the lane's D accumulators;
//   3. lanes are brought to the wave's reference and summed by a butterfly,
//      waves combined through LDS: (max, sum, o).
// With several splits the partials are merged by the plain log-sum-exp
// merge; with one the block writes o / sum.
#include "device.hpp"
#include "kernels.hpp"

namespace lkv {
namespace {

constexpr int kThreads = 256;
constexpr int kSplitWaves = 8;
constexpr float kSlack = 8.0f;       // decode: a lane's weights stay below e^kSlack
constexpr int kSplitThreads = 64 * kSplitWaves;

// Encode: kSub threads per (sequence, new token, head), a block per
// 256 / kSub of them and per channel group (blockIdx.y); blockIdx.z = 0
// keys, 1 values.  Nearest codeword in squared distance, fp32, ties to the
// lowest index: each of the kSub threads scans 256 / kSub consecutive codes,
// then the kSub candidates are compared (equal distances: lower code).
// kSub = 4 when few tokens are coded, so that the grid fills the chip.
template <int D, int R, int kSub>
__global__ __launch_bounds__(kThreads) void vq_encode_kernel(VqArgs a) {
  constexpr int G = D / kVqSub;
  constexpr int J = kVqSub * R;
  __shared__ float cw[kVqCodes * J];
  const int j = blockIdx.y;
  const bool is_v = blockIdx.z == 1;
  // codebook [R][256][G][4]: codeword c of group j is loop r's 4 channels at
  // ((r * 256 + c) * G + j) * 4, r = 0 .. R-1
  const uint16_t* cb = is_v ? a.cb_v : a.cb_k;
  for (int e = threadIdx.x; e < kVqCodes * R; e += kThreads) {     // one (code, loop) slice each
    const int c = e / R, r = e % R;
    const uint2 w = *reinterpret_cast<const uint2*>(cb + ((static_cast<int64_t>(r) * kVqCodes + c) * G + j) * kVqSub);
    float* d = cw + c * J + kVqSub * r;
    d[0] = f16_to_f32(w.x & 0xffffu);
    d[1] = f16_to_f32(w.x >> 16);
    d[2] = f16_to_f32(w.y & 0xffffu);
    d[3] = f16_to_f32(w.y >> 16);
  }
  __syncthreads();

  const int64_t m = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / kSub;
  const int sub = threadIdx.x % kSub;
  const int64_t M = static_cast<int64_t>(a.batch) * a.n_new * a.H;
  if (m >= M) return;                       // the kSub threads of m leave together
  const int h = static_cast<int>(m % a.H);
  const int64_t bi = m / a.H;
  const int i = static_cast<int>(bi % a.n_new);
  const int b = static_cast<int>(bi / a.n_new);
  const uint16_t* src = is_v ? a.v_in : a.k_in;
  float x[J];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint16_t* row = src + (((static_cast<int64_t>(r) * a.batch + b) * a.n_new + i) * a.H + h) * D + kVqSub * j;
    const uint2 w = *reinterpret_cast<const uint2*>(row);
    x[kVqSub * r + 0] = bf16_to_f32(static_cast<uint16_t>(w.x & 0xffffu));
    x[kVqSub * r + 1] = bf16_to_f32(static_cast<uint16_t>(w.x >> 16));
    x[kVqSub * r + 2] = bf16_to_f32(static_cast<uint16_t>(w.y & 0xffffu));
    x[kVqSub * r + 3] = bf16_to_f32(static_cast<uint16_t>(w.y >> 16));
  }
  float best = INFINITY;
  int best_c = 0;
  constexpr int kSpan = kVqCodes / kSub;
  for (int c = sub * kSpan; c < (sub + 1) * kSpan; ++c) {
    float dist = 0.0f;
#pragma unroll
    for (int e = 0; e < J; ++e) {
      const float t = x[e] - cw[c * J + e];
      dist = fmaf(t, t, dist);
    }
    if (dist < best) {
      best = dist;
      best_c = c;
    }
  }
#pragma unroll
  for (int o = 1; o < kSub; o <<= 1) {
    const float ob = __shfl_xor(best, o, 64);
    const int oc = __shfl_xor(best_c, o, 64);
    if (ob < best || (ob == best && oc < best_c)) {
      best = ob;
      best_c = oc;
    }
  }
  if (sub != 0) return;
  const int t = a.seq_lens[b] + i;
  const int32_t page = a.block_tables[static_cast<int64_t>(b) * a.max_pages + t / a.P];
  const int64_t hb = static_cast<int64_t>(2) * a.P * G;
  uint8_t* blk = a.pool + (static_cast<int64_t>(h) * a.num_pages + page) * hb;
  // byte j ^ (t mod G) of the row (XOR-rotated by the token's position)
  blk[(is_v ? a.P * G : 0) + (t % a.P) * G + (j ^ (t % G))] = static_cast<uint8_t>(best_c);
}

// Split pass of the decode of loop a.loop: one block of kSplitWaves waves
// per (split, head, sequence).  After the block has built its two tables,
// every wave streams its own 64-token tiles (tiles w, w + kSplitWaves, ...
// of the split) with a private online softmax and no barrier: lane = token;
// the key row gives the score by D/4 table reads; a running wave maximum
// rescales the lane's D accumulators only when it rises; the value row adds
// p * (codeword slice) group by group.  The next tile's rows are loaded
// while the current one is used.
//
// Bank-conflict-free lookups.  Index bytes are stored XOR-rotated: byte r
// of token t's row names group r ^ (t mod G) (G = D/4 groups), and a tile
// starts at a multiple of 64, so at step r lane i reads group r ^ (i mod G).
// The tables are code-major: entry (code, column) at code * 256 bytes +
// column * (4 or 8), column c holding group c mod G, and lane i uses column
// (r ^ (i mod G)) + G * (i / G) (values: modulo 32 columns).  The 64 lanes
// of a key read (32 of a value read) then address distinct banks whatever
// the codes.  One v_perm builds an address from the code byte and a per-lane
// column byte.  Value accumulator slot r of lane i holds group r ^ (i mod G);
// the lane butterfly undoes this for free: at lane bit m < G both partners
// keep the slots with bit m clear, and a lane ends with group i mod G.
template <int D, int R>
__global__ __launch_bounds__(kSplitThreads) void vq_split_kernel(VqArgs a) {
  constexpr int G = D / kVqSub;          // groups = index bytes per row (16 or 32)
  constexpr int kWords = G / 16;         // 16-byte words per index row
  constexpr int kKeyCols = 64;           // 4-byte key-table columns per code (256 B)
  constexpr int kValCols = 32;           // 8-byte value-table columns per code (256 B)
  constexpr int kValRegs = (G + 2) / 3;  // column registers of the value table (3 columns each)
  // key table at LDS 0 (addresses < 64 KB), value table at 64 KB: its
  // addresses carry 0x01 in byte 2, supplied by the column register
  constexpr int kLut = kVqCodes * kKeyCols * 4, kCvs = kVqCodes * kValCols * 8;
  constexpr int kOut = kSplitWaves * D * 4;
  static_assert(kLut == 65536, "value table must start at 64 KB");
  __shared__ __align__(16) unsigned char smem[kLut + kCvs + kOut + 2 * kSplitWaves * 4];
  float* lut = reinterpret_cast<float*>(smem);
  uint2* cvs = reinterpret_cast<uint2*>(smem + kLut);      // value codeword slices of the loop (4 x fp16)
  float* wout = reinterpret_cast<float*>(smem + kLut + kCvs);
  float* wmax = wout + kSplitWaves * D;
  float* wsum = wmax + kSplitWaves;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int T = a.seq_lens[b];
  const int start = split * a.split_len;
  const int end = min(start + a.split_len, T);
  const int64_t pair = static_cast<int64_t>(b) * a.H + h;
  if (start >= end) {
    if (a.S == 1 && tid < D) a.out[pair * D + tid] = 0.0f;     // empty sequence
    return;
  }

  const int lgP = __builtin_ctz(static_cast<unsigned>(a.P));
  const int pmask = a.P - 1;
  const int64_t hb = static_cast<int64_t>(2) * a.P * G;
  const uint8_t* head = a.pool + static_cast<int64_t>(h) * a.num_pages * hb;
  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_pages;
  const int n_tiles = (end - start + 63) >> 6;

  // a lane past the end (or a tile past the split) stands for the split's
  // last token, whose score is then masked.  Rows are requested two tiles
  // ahead (three register buffers, so no buffer is copied and a load is
  // waited for only where its rows are used), and the physical page of a
  // tile's token one tile before its rows.
  auto token = [&](int tile) { return min(start + 64 * tile + lane, end - 1); };
  auto page_of = [&](int tile) { return bt[token(tile) >> lgP]; };
  auto load_rows = [&](uint4 (&kr)[kWords], uint4 (&vr)[kWords], int tile, int32_t page) {
    const uint8_t* row = head + static_cast<int64_t>(page) * hb + (token(tile) & pmask) * G;
#pragma unroll
    for (int k = 0; k < kWords; ++k) {
      kr[k] = reinterpret_cast<const uint4*>(row)[k];
      vr[k] = reinterpret_cast<const uint4*>(row + a.P * G)[k];
    }
  };
  uint4 kb0[kWords], vb0[kWords], kb1[kWords], vb1[kWords], kb2[kWords], vb2[kWords];
  int32_t pg0 = 0, pg1 = 0, pg2 = page_of(wave + 2 * kSplitWaves);
  load_rows(kb0, vb0, wave, page_of(wave));
  load_rows(kb1, vb1, wave + kSplitWaves, page_of(wave + kSplitWaves));

  // tables from the loop's codeword slices, [256 codes][G groups][4] fp16
  // contiguous in each codebook; every load is issued before the first use
  {
    const int64_t slice = static_cast<int64_t>(a.loop) * kVqCodes * G * kVqSub;
    // keys: a wave step covers codes c, c + 1 (lane halves); lane column
    // g = lane & 31 (group g mod G) and its copy g + 32 get q_g . codeword
    const int gk = lane & 31, jk = gk & (G - 1), half = lane >> 5;
    const uint2 qw = *reinterpret_cast<const uint2*>(a.q + pair * D + kVqSub * jk);
    const float q0 = bf16_to_f32(static_cast<uint16_t>(qw.x & 0xffffu)) * a.sm_scale;
    const float q1 = bf16_to_f32(static_cast<uint16_t>(qw.x >> 16)) * a.sm_scale;
    const float q2 = bf16_to_f32(static_cast<uint16_t>(qw.y & 0xffffu)) * a.sm_scale;
    const float q3 = bf16_to_f32(static_cast<uint16_t>(qw.y >> 16)) * a.sm_scale;
    constexpr int kKeySteps = kVqCodes / 2 / kSplitWaves;       // 16
    uint2 kc[kKeySteps];
#pragma unroll
    for (int u = 0; u < kKeySteps; ++u) {
      const int code = 2 * (wave + kSplitWaves * u) + half;
      kc[u] = *reinterpret_cast<const uint2*>(a.cb_k + slice + (code * G + jk) * kVqSub);
    }
    // values: 16-byte chunks (two groups) copied to column g and its copies
    constexpr int kChunks = kVqCodes * G / 2;                  // 16-byte chunks of the slice
    constexpr int kValSteps = kChunks / kSplitThreads;
    uint4 vc[kValSteps];
#pragma unroll
    for (int u = 0; u < kValSteps; ++u)
      vc[u] = reinterpret_cast<const uint4*>(a.cb_v + slice)[u * kSplitThreads + tid];
#pragma unroll
    for (int u = 0; u < kKeySteps; ++u) {
      const int code = 2 * (wave + kSplitWaves * u) + half;
      float e = q0 * f16_to_f32(kc[u].x & 0xffffu);
      e = fmaf(q1, f16_to_f32(kc[u].x >> 16), e);
      e = fmaf(q2, f16_to_f32(kc[u].y & 0xffffu), e);
      e = fmaf(q3, f16_to_f32(kc[u].y >> 16), e);
      // the lane halves write opposite column halves first: distinct banks
      lut[code * kKeyCols + gk + 32 * half] = e;
      lut[code * kKeyCols + gk + 32 * (1 - half)] = e;
    }
#pragma unroll
    for (int u = 0; u < kValSteps; ++u) {
      const int ch = u * kSplitThreads + tid;
      const int code = ch / (G / 2), g0 = 2 * (ch % (G / 2));
#pragma unroll
      for (int m = 0; m < kValCols / G; ++m)
        *reinterpret_cast<uint4*>(cvs + code * kValCols + g0 + G * m) = vc[u];
    }
  }

  // per-lane column bytes: key columns four to a register, value columns
  // three to a register with 0x01 (the table's 64 KB base) in byte 3
  const int ig = lane & (G - 1);
  uint32_t kcol[G / 4], vcol[kValRegs];
#pragma unroll
  for (int m = 0; m < G / 4; ++m) {
    uint32_t w = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) w |= static_cast<uint32_t>((((4 * m + u) ^ ig) + G * ((lane / G) & (kKeyCols / G - 1))) * 4) << (8 * u);
    kcol[m] = w;
  }
#pragma unroll
  for (int m = 0; m < kValRegs; ++m) {
    uint32_t w = 0x01000000u;
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int r = min(3 * m + u, G - 1);
      w |= static_cast<uint32_t>((((r ^ ig) + G * ((lane / G) & (kValCols / G - 1))) * 8) & 0xff) << (8 * u);
    }
    vcol[m] = w;
  }
  __syncthreads();

  float acc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) acc[i] = 0.0f;
  float M = -INFINITY, lsum = 0.0f;

  // one tile: the page three tiles ahead and the rows two tiles ahead are
  // requested first
  auto step = [&](const uint4 (&kr)[kWords], const uint4 (&vr)[kWords], uint4 (&kn)[kWords],
                  uint4 (&vn)[kWords], int32_t pg_use, int32_t& pg_load, int tile) {
    pg_load = page_of(tile + 3 * kSplitWaves);
    load_rows(kn, vn, tile + 2 * kSplitWaves, pg_use);
    const int t = start + 64 * tile + lane;
    // score: D/4 table reads, four partial sums
    float sp[4];
#pragma unroll
    for (int k = 0; k < kWords; ++k) {
      const uint32_t ws[4] = {kr[k].x, kr[k].y, kr[k].z, kr[k].w};
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = 16 * k + q;
        // byte 0: column (register byte r % 4), byte 1: code (word byte q % 4)
        const uint32_t addr = __builtin_amdgcn_perm(ws[q / 4], kcol[r / 4], 0x0c0c0000u | ((4u + q % 4) << 8) | (r % 4));
        const float e = *reinterpret_cast<const float*>(smem + addr);
        if (k == 0 && q < 4) sp[q] = e;
        else sp[q % 4] += e;
      }
    }
    const float s = (sp[0] + sp[1]) + (sp[2] + sp[3]);
    const bool valid = t < end;
    // the lane's reference M moves up only when a score passes it by more
    // than kSlack (weights stay below e^kSlack); rare after the first tile
    const bool raise = valid && s > M + kSlack;
    if (__any(raise)) {
      const float alpha = raise ? __expf(M - s) : 1.0f;   // 0 for the lane's first score
#pragma unroll
      for (int i = 0; i < D; ++i) acc[i] *= alpha;
      lsum *= alpha;
      M = raise ? s : M;
    }
    const float p = valid ? __expf(s - M) : 0.0f;
    lsum += p;
#pragma unroll
    for (int k = 0; k < kWords; ++k) {
      const uint32_t ws[4] = {vr[k].x, vr[k].y, vr[k].z, vr[k].w};
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = 16 * k + q;
        // byte 0: column, byte 1: code, byte 2: 0x01 (64 KB), byte 3: 0
        const uint32_t addr = __builtin_amdgcn_perm(ws[q / 4], vcol[r / 3], 0x0c030000u | ((4u + q % 4) << 8) | (r % 3));
        const uint2 cw = *reinterpret_cast<const uint2*>(smem + addr);
        acc[4 * r + 0] = fmaf(p, f16_to_f32(cw.x & 0xffffu), acc[4 * r + 0]);
        acc[4 * r + 1] = fmaf(p, f16_to_f32(cw.x >> 16), acc[4 * r + 1]);
        acc[4 * r + 2] = fmaf(p, f16_to_f32(cw.y & 0xffffu), acc[4 * r + 2]);
        acc[4 * r + 3] = fmaf(p, f16_to_f32(cw.y >> 16), acc[4 * r + 3]);
      }
    }
  };
  const int n_steps = wave < n_tiles ? (n_tiles - wave + kSplitWaves - 1) / kSplitWaves : 0;
  int tile = wave, i = 0;
  for (; i + 3 <= n_steps; i += 3, tile += 3 * kSplitWaves) {
    step(kb0, vb0, kb2, vb2, pg2, pg0, tile);
    step(kb1, vb1, kb0, vb0, pg0, pg1, tile + kSplitWaves);
    step(kb2, vb2, kb1, vb1, pg1, pg2, tile + 2 * kSplitWaves);
  }
  if (i < n_steps) step(kb0, vb0, kb2, vb2, pg2, pg0, tile);
  if (i + 1 < n_steps) step(kb1, vb1, kb0, vb0, pg0, pg1, tile + kSplitWaves);

  // common reference of the wave: the lanes' accumulators are rescaled to
  // the largest lane reference (a lane without tokens has M = -inf and zeros)
  {
    const float mw = dpp_wave_max(M);
    const float f = M == -INFINITY ? 0.0f : __expf(M - mw);
#pragma unroll
    for (int i = 0; i < D; ++i) acc[i] *= f;
    lsum *= f;
    M = mw;
  }

  // lane butterfly: at lane bit m < G both partners keep the slots with bit
  // m clear (slot s of lane i holds group s ^ (i mod G), so the partner holds
  // the same group in slot s ^ m); then lanes of equal i mod G are added
#pragma unroll
  for (int m = 1; m < G; m <<= 1) {
#pragma unroll
    for (int s = 0; s < G; ++s) {
      if (s & (2 * m - 1)) continue;        // slots still held have their lower bits clear
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[4 * s + c] += __shfl_xor(acc[4 * (s + m) + c], m, 64);
    }
  }
#pragma unroll
  for (int m = G; m < 64; m <<= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] += __shfl_xor(acc[c], m, 64);
  }
  lsum = wave_sum(lsum);
  if (lane < G) {
#pragma unroll
    for (int c = 0; c < 4; ++c) wout[wave * D + 4 * lane + c] = acc[c];
  }
  if (lane == 0) {
    wmax[wave] = M;
    wsum[wave] = lsum;
  }
  __syncthreads();
  if (tid < D) {
    float mb = wmax[0];
#pragma unroll
    for (int w = 1; w < kSplitWaves; ++w) mb = fmaxf(mb, wmax[w]);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) {
      const float f = __expf(wmax[w] - mb);   // 0 for a wave without tiles
      o = fmaf(f, wout[w * D + tid], o);
      l = fmaf(f, wsum[w], l);
    }
    if (a.S == 1) {
      a.out[pair * D + tid] = o / l;
    } else {
      float* part = a.partials + (pair * a.S + split) * (D + kPartialPad);
      part[kPartialPad + tid] = o;
      if (tid == 0) {
        part[0] = mb;
        part[1] = l;
      }
    }
  }
}

template <int D, int R>
hipError_t launch_encode_t(const VqArgs& a, hipStream_t stream) {
  const int64_t M = static_cast<int64_t>(a.batch) * a.n_new * a.H;
  const ProfEvents ev = prof_events(kClassAppend);
  if (M <= 16384) {                        // few token-heads (a decode step): four threads each
    constexpr int kPer = kThreads / 4;
    const dim3 grid(static_cast<unsigned>((M + kPer - 1) / kPer), D / kVqSub, 2);
    hipExtLaunchKernelGGL((vq_encode_kernel<D, R, 4>), grid, dim3(kThreads), 0, stream, ev.start, ev.stop, 0, a);
  } else {
    const dim3 grid(static_cast<unsigned>((M + kThreads - 1) / kThreads), D / kVqSub, 2);
    hipExtLaunchKernelGGL((vq_encode_kernel<D, R, 1>), grid, dim3(kThreads), 0, stream, ev.start, ev.stop, 0, a);
  }
  return hipGetLastError();
}

template <int D, int R>
hipError_t launch_split_t(const VqArgs& a, hipStream_t stream) {
  const ProfEvents ev = prof_events(kClassSplit);
  hipExtLaunchKernelGGL((vq_split_kernel<D, R>), dim3(a.S, a.H, a.batch), dim3(kSplitThreads), 0, stream,
                        ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_encode_d(const VqArgs& a, hipStream_t stream) {
  switch (a.R) {
    case 2: return launch_encode_t<D, 2>(a, stream);
    case 3: return launch_encode_t<D, 3>(a, stream);
    default: return launch_encode_t<D, 4>(a, stream);
  }
}

template <int D>
hipError_t launch_split_d(const VqArgs& a, hipStream_t stream) {
  switch (a.R) {
    case 2: return launch_split_t<D, 2>(a, stream);
    case 3: return launch_split_t<D, 3>(a, stream);
    default: return launch_split_t<D, 4>(a, stream);
  }
}

}  // namespace

hipError_t launch_vq_encode(const VqArgs& a, int D, hipStream_t stream) {
  return D == 128 ? launch_encode_d<128>(a, stream) : launch_encode_d<64>(a, stream);
}

hipError_t launch_vq_split(const VqArgs& a, int D, hipStream_t stream) {
  return D == 128 ? launch_split_d<128>(a, stream) : launch_split_d<64>(a, stream);
}

}  // namespace lkv
