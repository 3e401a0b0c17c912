// vq.hip -- joint vector quantization of keys and values across loop steps,
// and the split pass of decode attention over such a cache (LoopVQ-style).
//
// Source: "LoopVQ: Sub 1-bit KV Cache Quantization for Looped
// Transformers", abstract (概要): the KV cache of a looped model is
// redundant along the loop axis; LoopVQ codes channels of several loop
// steps jointly with codebooks and reaches 0.5 bit per element.
//
// Format: for one layer, token and head, channel group j's joint vector is
// the concatenation over loops r of channels [4j, 4j+4) of loop r's key (or
// value), 4R numbers; group j's codebook holds 256 codewords (fp16), so one
// byte codes 4R elements (R = 4: 0.5 bit per element).  All loops of a
// layer share one index cache; loop r decodes slice [4r, 4r+4) of each
// codeword.
//
// Layout of a head-block (one head, one page of P tokens): P key index
// rows of D/4 bytes, then P value index rows of D/4 bytes (token-major), so
// the 64 lanes of a wave read one 64-token tile's rows as contiguous runs.
//
// Decode of loop r, one block of 8 waves per (split, head, sequence):
//   1. a table lut[j][c] = sm_scale * q[4j..4j+4) . key codeword_c[4r..4r+4)
//      and the loop's value codeword slices, both in LDS, so a token's score
//      is the sum of D/4 table reads addressed by its key bytes;
//   2. each wave streams its own 64-token tiles (lane = token) with a
//      private online softmax: score, wave maximum (accumulators rescaled
//      only when it rises), p_t, and per value group one LDS read of the 4
//      fp16 channels of the chosen codeword and 4 FMAs into the lane's D
//      accumulators;
//   3. lanes are summed by a butterfly, waves through LDS: (max, sum, o).
// With several splits the partials are merged by the plain log-sum-exp
// merge; with one the block writes o / sum.
#include "device.hpp"
#include "kernels.hpp"

namespace lkv {
namespace {

constexpr int kThreads = 256;
constexpr int kSplitWaves = 8;
constexpr int kSplitThreads = 64 * kSplitWaves;

// Encode: one thread per (sequence, new token, head), a block per 256 of
// them and per channel group (blockIdx.y); blockIdx.z = 0 keys, 1 values.
// Nearest codeword in squared distance, fp32, ties to the lowest index.
template <int D, int R>
__global__ __launch_bounds__(kThreads) void vq_encode_kernel(VqArgs a) {
  constexpr int G = D / kVqSub;
  constexpr int J = kVqSub * R;
  __shared__ float cw[kVqCodes * J];
  const int j = blockIdx.y;
  const bool is_v = blockIdx.z == 1;
  const uint16_t* cb = (is_v ? a.cb_v : a.cb_k) + static_cast<int64_t>(j) * kVqCodes * J;
  for (int e = threadIdx.x; e < kVqCodes * J; e += kThreads) cw[e] = f16_to_f32(cb[e]);
  __syncthreads();

  const int64_t m = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t M = static_cast<int64_t>(a.batch) * a.n_new * a.H;
  if (m >= M) return;
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
  for (int c = 0; c < kVqCodes; ++c) {
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
  const int t = a.seq_lens[b] + i;
  const int32_t page = a.block_tables[static_cast<int64_t>(b) * a.max_pages + t / a.P];
  const int64_t hb = static_cast<int64_t>(2) * a.P * G;
  uint8_t* blk = a.pool + (static_cast<int64_t>(h) * a.num_pages + page) * hb;
  blk[(is_v ? a.P * G : 0) + (t % a.P) * G + j] = static_cast<uint8_t>(best_c);
}

// Split pass of the decode of loop a.loop: one block of kSplitWaves waves
// per (split, head, sequence).  After the block has built its two tables,
// every wave streams its own 64-token tiles (tiles w, w + kSplitWaves, ...
// of the split) with a private online softmax and no barrier: lane = token;
// the key row gives the score by D/4 table reads; a running wave maximum
// rescales the lane's D accumulators only when it rises; the value row adds
// p * (codeword slice) group by group.  The next tile's rows are loaded
// while the current one is used.  At the end the lanes of a wave are summed
// by a butterfly (each lane keeps D/64 channels) and the waves are combined
// through LDS with their maxima.  With one split the block writes the
// normalized output itself.
template <int D, int R>
__global__ __launch_bounds__(kSplitThreads) void vq_split_kernel(VqArgs a) {
  constexpr int G = D / kVqSub;      // index bytes per row
  constexpr int J = kVqSub * R;
  constexpr int kWords = G / 16;     // 16-byte words per index row
  constexpr int kKeep = D / 64;      // channels a lane holds after the butterfly
  // one LDS block, score table first: its row offsets (and those of the
  // first 64 KB of codeword slices) fit the LDS instructions' 16-bit offset
  constexpr int kLut = G * kVqCodes * 4, kCvs = G * kVqCodes * 8, kOut = kSplitWaves * D * 4;
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

  // key and value index rows of this lane's token in one tile; a lane past
  // the end (or a tile past the split) reads the split's last token, whose
  // score is then masked
  auto load_rows = [&](uint4 (&kr)[kWords], uint4 (&vr)[kWords], int tile) {
    const int t = min(start + 64 * tile + lane, end - 1);
    const uint8_t* row = head + static_cast<int64_t>(bt[t >> lgP]) * hb + (t & pmask) * G;
#pragma unroll
    for (int k = 0; k < kWords; ++k) {
      kr[k] = reinterpret_cast<const uint4*>(row)[k];
      vr[k] = reinterpret_cast<const uint4*>(row + a.P * G)[k];
    }
  };
  uint4 kr[kWords], vr[kWords];
  load_rows(kr, vr, wave);

  // score table and value codeword slices (thread = codeword; all loads of a
  // batch of groups issued before use)
  {
    const int c = tid & (kVqCodes - 1);
    constexpr int kStep = kSplitThreads / kVqCodes;
    constexpr int kBatch = 4;
    for (int j0 = tid / kVqCodes; j0 < G; j0 += kStep * kBatch) {
      uint2 qw[kBatch], kc[kBatch], vc[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int j = min(j0 + kStep * u, G - 1);
        const int64_t cwo = (static_cast<int64_t>(j) * kVqCodes + c) * J + kVqSub * a.loop;
        qw[u] = *reinterpret_cast<const uint2*>(a.q + pair * D + kVqSub * j);
        kc[u] = *reinterpret_cast<const uint2*>(a.cb_k + cwo);
        vc[u] = *reinterpret_cast<const uint2*>(a.cb_v + cwo);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int j = j0 + kStep * u;
        if (j >= G) break;
        float s = bf16_to_f32(static_cast<uint16_t>(qw[u].x & 0xffffu)) * f16_to_f32(kc[u].x & 0xffffu);
        s = fmaf(bf16_to_f32(static_cast<uint16_t>(qw[u].x >> 16)), f16_to_f32(kc[u].x >> 16), s);
        s = fmaf(bf16_to_f32(static_cast<uint16_t>(qw[u].y & 0xffffu)), f16_to_f32(kc[u].y & 0xffffu), s);
        s = fmaf(bf16_to_f32(static_cast<uint16_t>(qw[u].y >> 16)), f16_to_f32(kc[u].y >> 16), s);
        lut[j * kVqCodes + c] = s * a.sm_scale;
        cvs[j * kVqCodes + c] = vc[u];
      }
    }
  }
  __syncthreads();

  float acc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) acc[i] = 0.0f;
  float M = -INFINITY, lsum = 0.0f;

  for (int tile = wave; tile < n_tiles; tile += kSplitWaves) {
    uint4 kn[kWords], vn[kWords];
    load_rows(kn, vn, tile + kSplitWaves);
    const int t = start + 64 * tile + lane;
    // score: D/4 table reads, four partial sums
    float sp[4];
#pragma unroll
    for (int k = 0; k < kWords; ++k) {
      const uint32_t ws[4] = {kr[k].x, kr[k].y, kr[k].z, kr[k].w};
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        // byte offset of the entry in its row; kept opaque so that the row's
        // offset goes into the LDS instruction's immediate field
        uint32_t off = ((ws[q / 4] >> (8 * (q % 4))) & 0xffu) << 2;
        asm volatile("" : "+v"(off));
        const float e = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(lut + (16 * k + q) * kVqCodes) + off);
        if (k == 0 && q < 4) sp[q] = e;
        else sp[q % 4] += e;
      }
    }
    const float s = t < end ? (sp[0] + sp[1]) + (sp[2] + sp[3]) : -INFINITY;
    const float mt = dpp_wave_max(s);      // wave-uniform; finite (lane 0 is in range)
    if (mt > M) {
      const float alpha = __expf(M - mt);  // 0 on the first tile
#pragma unroll
      for (int i = 0; i < D; ++i) acc[i] *= alpha;
      lsum *= alpha;
      M = mt;
    }
    const float p = __expf(s - M);         // 0 past the end
    lsum += p;
#pragma unroll
    for (int k = 0; k < kWords; ++k) {
      const uint32_t ws[4] = {vr[k].x, vr[k].y, vr[k].z, vr[k].w};
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int g = 16 * k + q;
        const uint2 cw = cvs[g * kVqCodes + ((ws[q / 4] >> (8 * (q % 4))) & 0xffu)];
        acc[4 * g + 0] = fmaf(p, f16_to_f32(cw.x & 0xffffu), acc[4 * g + 0]);
        acc[4 * g + 1] = fmaf(p, f16_to_f32(cw.x >> 16), acc[4 * g + 1]);
        acc[4 * g + 2] = fmaf(p, f16_to_f32(cw.y & 0xffffu), acc[4 * g + 2]);
        acc[4 * g + 3] = fmaf(p, f16_to_f32(cw.y >> 16), acc[4 * g + 3]);
      }
    }
#pragma unroll
    for (int k = 0; k < kWords; ++k) {
      kr[k] = kn[k];
      vr[k] = vn[k];
    }
  }

  // butterfly over the lanes: at the step of lane bit m, a lane keeps the
  // upper half of its channels if its bit m is set, else the lower half, and
  // adds its partner's copy of that half.
#pragma unroll
  for (int m = 32, n = D; m > 0; m >>= 1, n >>= 1) {
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      const float send = upper ? acc[i] : acc[i + n / 2];
      const float keep = upper ? acc[i + n / 2] : acc[i];
      acc[i] = keep + __shfl_xor(send, m, 64);
    }
  }
  lsum = wave_sum(lsum);
  // channel of acc[i] after the butterfly: i + sum over lane bits m of (bit set) * D / (128 / m)
  int base = 0;
#pragma unroll
  for (int m = 32, n = D / 2; m > 0; m >>= 1, n >>= 1)
    if (lane & m) base += n;
#pragma unroll
  for (int i = 0; i < kKeep; ++i) wout[wave * D + base + i] = acc[i];
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
  const dim3 grid(static_cast<unsigned>((M + kThreads - 1) / kThreads), D / kVqSub, 2);
  hipLaunchKernelGGL((vq_encode_kernel<D, R>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D, int R>
hipError_t launch_split_t(const VqArgs& a, hipStream_t stream) {
  prof_mark(kClassSplit, 0, stream);
  hipLaunchKernelGGL((vq_split_kernel<D, R>), dim3(a.S, a.H, a.batch), dim3(kSplitThreads), 0, stream, a);
  const hipError_t e = hipGetLastError();
  prof_mark(kClassSplit, 1, stream);
  return e;
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
  prof_mark(kClassAppend, 0, stream);
  const hipError_t e = D == 128 ? launch_encode_d<128>(a, stream) : launch_encode_d<64>(a, stream);
  prof_mark(kClassAppend, 1, stream);
  return e;
}

hipError_t launch_vq_split(const VqArgs& a, int D, hipStream_t stream) {
  return D == 128 ? launch_split_d<128>(a, stream) : launch_split_d<64>(a, stream);
}

}  // namespace lkv
