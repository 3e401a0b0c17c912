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
// rows of D/4 bytes (token-major), then the value indices in four chunks of
// D/16 groups each, chunk-major: [4][P][D/16] bytes, so the wave that owns a
// chunk reads its bytes of 64 tokens as one contiguous run.
//
// Decode of loop r, one 512-thread block (8 waves) per (split, head,
// sequence), a split streamed in chunks of 1024 tokens:
//   1. a table lut[j][c] = sm_scale * q[4j..4j+4) . key codeword_c[4r..4r+4)
//      and the loop's value codeword slices, both in LDS, so a token's score
//      is the sum of D/4 table reads addressed by its key bytes;
//   2. the chunk's scores and maximum (running max across chunks);
//   3. wave w owns value chunk w % 4 and every other 64-token tile: per
//      token p_t = exp(s_t - max) and, per group of the chunk, one LDS read
//      of the 4 fp16 channels of the chosen codeword and 4 FMAs;
//   4. lanes, then the two waves of a chunk, are summed: (max, sum, o).
// The partials are merged by the plain log-sum-exp merge.
#include "device.hpp"
#include "kernels.hpp"

namespace lkv {
namespace {

constexpr int kThreads = 256;
constexpr int kTokPerThread = 4;     // tokens per thread per step (loads in flight)

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
  if (is_v) {
    constexpr int kCg = G / 4;     // groups per value chunk
    blk[a.P * G + ((j / kCg) * a.P + t % a.P) * kCg + j % kCg] = static_cast<uint8_t>(best_c);
  } else {
    blk[(t % a.P) * G + j] = static_cast<uint8_t>(best_c);
  }
}

// Split pass of the decode of loop a.loop: a block streams its split in
// chunks of kVqChunk tokens with an online softmax (running max and sum;
// accumulators rescaled when the max rises).  The key rows of the next chunk
// and the value bytes of the next tile are loaded before the current ones
// are used.
constexpr int kSplitThreads = 512;
template <int D, int R>
__global__ __launch_bounds__(kSplitThreads) void vq_split_kernel(VqArgs a) {
  constexpr int G = D / kVqSub;      // index bytes per key row
  constexpr int J = kVqSub * R;
  constexpr int kWords = G / 16;     // 16-byte words per key row
  constexpr int kCg = G / 4;         // groups per value chunk
  constexpr int kAcc = kVqSub * kCg; // channels per value chunk
  constexpr int kTok = kVqChunk / kSplitThreads;   // tokens per thread per score pass
  __shared__ float lut[G * kVqCodes];
  __shared__ uint2 cvs[G * kVqCodes];     // value codeword slices of the loop (4 x fp16)
  __shared__ float sc[kVqChunk];
  __shared__ float red[kSplitThreads / 64];
  __shared__ float ored[4 * kAcc];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int T = a.seq_lens[b];
  const int start = split * a.split_len;
  const int end = min(start + a.split_len, T);
  if (start >= end) return;
  const int64_t pair = static_cast<int64_t>(b) * a.H + h;

  const int lgP = __builtin_ctz(static_cast<unsigned>(a.P));
  const int pmask = a.P - 1;
  const int64_t hb = static_cast<int64_t>(2) * a.P * G;
  const uint8_t* head = a.pool + static_cast<int64_t>(h) * a.num_pages * hb;
  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_pages;

  // key rows of one chunk, kTok per thread
  auto load_keys = [&](uint4 (&w)[kTok][kWords], int c0) {
#pragma unroll
    for (int u = 0; u < kTok; ++u) {
      const int t = c0 + u * kSplitThreads + tid;
#pragma unroll
      for (int k = 0; k < kWords; ++k) {
        w[u][k] = make_uint4(0u, 0u, 0u, 0u);
        if (t < end)
          w[u][k] = reinterpret_cast<const uint4*>(head + static_cast<int64_t>(bt[t >> lgP]) * hb + (t & pmask) * G)[k];
      }
    }
  };
  uint4 kw[kTok][kWords];
  load_keys(kw, start);

  // 1. score table and value codeword slices (thread = codeword; all loads of
  //    a batch of groups issued before use)
  {
    const int c = tid & (kVqCodes - 1);
    constexpr int kStep = kSplitThreads / kVqCodes;     // 2
    constexpr int kBatch = 4;
    for (int j0 = tid >> 8; j0 < G; j0 += kStep * kBatch) {
      uint2 qw[kBatch], kc[kBatch], vc[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int j = j0 + kStep * u;
        const int64_t cwo = (static_cast<int64_t>(j) * kVqCodes + c) * J + kVqSub * a.loop;
        qw[u] = *reinterpret_cast<const uint2*>(a.q + pair * D + kVqSub * j);
        kc[u] = *reinterpret_cast<const uint2*>(a.cb_k + cwo);
        vc[u] = *reinterpret_cast<const uint2*>(a.cb_v + cwo);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int j = j0 + kStep * u;
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

  const int chunk = wave & 3, half = wave >> 2;   // value chunk and tile parity of this wave
  constexpr int kTiles = kVqChunk / 128;          // value tiles of a wave per chunk
  // value bytes of this wave's tiles of one chunk (lane = token slot)
  auto load_vals = [&](uint2 (&v)[kTiles], int c0) {
    const int c1 = min(c0 + kVqChunk, end);
#pragma unroll
    for (int i = 0; i < kTiles; ++i) {
      const int t = c0 + 64 * half + 128 * i + lane;
      v[i] = make_uint2(0u, 0u);
      if (t < c1) {
        const uint8_t* vb = head + static_cast<int64_t>(bt[t >> lgP]) * hb + a.P * G + (chunk * a.P + (t & pmask)) * kCg;
        if (kCg == 8) v[i] = *reinterpret_cast<const uint2*>(vb);
        else v[i].x = *reinterpret_cast<const uint32_t*>(vb);
      }
    }
  };
  uint2 vw[kTiles];
  load_vals(vw, start);
  float acc[kAcc];
#pragma unroll
  for (int i = 0; i < kAcc; ++i) acc[i] = 0.0f;
  float M = -INFINITY, lsum = 0.0f;

  for (int c0 = start; c0 < end; c0 += kVqChunk) {
    const int c1 = min(c0 + kVqChunk, end);
    // 2. scores of the chunk and its maximum
    float mloc = -INFINITY;
#pragma unroll
    for (int u = 0; u < kTok; ++u) {
      const int t = c0 + u * kSplitThreads + tid;
      float s = 0.0f;
#pragma unroll
      for (int k = 0; k < kWords; ++k) {
        const uint32_t ws[4] = {kw[u][k].x, kw[u][k].y, kw[u][k].z, kw[u][k].w};
#pragma unroll
        for (int q = 0; q < 16; ++q) s += lut[(16 * k + q) * kVqCodes + ((ws[q / 4] >> (8 * (q % 4))) & 0xffu)];
      }
      if (t < c1) {
        sc[t - c0] = s;
        mloc = fmaxf(mloc, s);
      }
    }
    // the next chunk's key rows and value bytes are in flight from here on
    uint2 vn[kTiles];
    if (c0 + kVqChunk < end) {
      load_keys(kw, c0 + kVqChunk);
      load_vals(vn, c0 + kVqChunk);
    }
    mloc = wave_max(mloc);
    if (lane == 0) red[wave] = mloc;
    __syncthreads();
    float mc = red[0];
#pragma unroll
    for (int i = 1; i < kSplitThreads / 64; ++i) mc = fmaxf(mc, red[i]);
    const float m_new = fmaxf(M, mc);
    const float alpha = __expf(M - m_new);                    // 0 on the first chunk
#pragma unroll
    for (int i = 0; i < kAcc; ++i) acc[i] *= alpha;
    lsum *= alpha;
    M = m_new;

    // 3. values: wave w owns chunk w % 4 and every other 64-token tile
#pragma unroll
    for (int i = 0; i < kTiles; ++i) {
      const int t = c0 + 64 * half + 128 * i + lane;
      if (t < c1) {
        const float p = __expf(sc[t - c0] - M);
        lsum += p;
        const uint32_t bytes[2] = {vw[i].x, vw[i].y};
#pragma unroll
        for (int g = 0; g < kCg; ++g) {
          const int code = (bytes[g / 4] >> (8 * (g % 4))) & 0xff;
          const uint2 cw = cvs[(kCg * chunk + g) * kVqCodes + code];
          acc[4 * g + 0] = fmaf(p, f16_to_f32(cw.x & 0xffffu), acc[4 * g + 0]);
          acc[4 * g + 1] = fmaf(p, f16_to_f32(cw.x >> 16), acc[4 * g + 1]);
          acc[4 * g + 2] = fmaf(p, f16_to_f32(cw.y & 0xffffu), acc[4 * g + 2]);
          acc[4 * g + 3] = fmaf(p, f16_to_f32(cw.y >> 16), acc[4 * g + 3]);
        }
      }
    }
    if (c0 + kVqChunk < end) {
#pragma unroll
      for (int i = 0; i < kTiles; ++i) vw[i] = vn[i];
    }
    __syncthreads();     // sc and red are rewritten by the next chunk
  }

  // 4. sums over lanes, then over the two waves of a chunk
#pragma unroll
  for (int i = 0; i < kAcc; ++i) acc[i] = wave_sum(acc[i]);
  lsum = wave_sum(lsum);
  if (half == 1) {
#pragma unroll
    for (int i = 0; i < kAcc; ++i)
      if (lane == i) ored[chunk * kAcc + i] = acc[i];
  }
  if (lane == 0 && chunk == 0) red[half] = lsum;
  __syncthreads();
  float* part = a.partials + (pair * a.S + split) * (D + kPartialPad);
  if (half == 0) {
#pragma unroll
    for (int i = 0; i < kAcc; ++i)
      if (lane == i) part[kPartialPad + kAcc * chunk + i] = acc[i] + ored[chunk * kAcc + i];
  }
  if (tid == 0) {
    part[0] = M;
    part[1] = red[0] + red[1];
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
