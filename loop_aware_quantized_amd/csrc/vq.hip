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
// Decode of loop r, one 256-thread block per (split, head, sequence):
//   1. a table lut[j][c] = sm_scale * q[4j..4j+4) . codeword_c[4r..4r+4) in
//      LDS (the query is fixed for the whole cache), so a token's score is
//      the sum of D/4 table reads addressed by its key bytes;
//   2. the split's scores and their maximum;
//   3. p_t = exp(s_t - max) added into a per-group histogram of value
//      codewords hist[j][c] (LDS float atomics: the order of additions, and
//      so the last bits of the output, may vary between runs);
//   4. o = sum_c hist[j][c] * value codeword_c[4r..4r+4) per group.
// The (max, sum, o) partials are merged by the plain log-sum-exp merge.
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
  blk[(is_v ? a.P * G : 0) + (t % a.P) * G + j] = static_cast<uint8_t>(best_c);
}

// Split pass of the decode of loop a.loop.
template <int D, int R>
__global__ __launch_bounds__(kThreads) void vq_split_kernel(VqArgs a) {
  constexpr int G = D / kVqSub;      // index bytes per token row
  constexpr int J = kVqSub * R;
  constexpr int kWords = G / 16;     // 16-byte words per row
  __shared__ float lut[G * kVqCodes];
  __shared__ float hist[G * kVqCodes];
  __shared__ float sc[kVqSplitMax];
  __shared__ float red[kThreads / 64];

  const int tid = threadIdx.x;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int T = a.seq_lens[b];
  const int start = split * a.split_len;
  const int end = min(start + a.split_len, T);
  if (start >= end) return;
  const int64_t pair = static_cast<int64_t>(b) * a.H + h;

  // 1. score table (thread = codeword) and a zero histogram
  {
    const int c = tid;
    for (int j = 0; j < G; ++j) {
      const uint2 qw = *reinterpret_cast<const uint2*>(a.q + pair * D + kVqSub * j);
      const uint2 cw = *reinterpret_cast<const uint2*>(a.cb_k + (static_cast<int64_t>(j) * kVqCodes + c) * J + kVqSub * a.loop);
      float s = bf16_to_f32(static_cast<uint16_t>(qw.x & 0xffffu)) * f16_to_f32(cw.x & 0xffffu);
      s = fmaf(bf16_to_f32(static_cast<uint16_t>(qw.x >> 16)), f16_to_f32(cw.x >> 16), s);
      s = fmaf(bf16_to_f32(static_cast<uint16_t>(qw.y & 0xffffu)), f16_to_f32(cw.y & 0xffffu), s);
      s = fmaf(bf16_to_f32(static_cast<uint16_t>(qw.y >> 16)), f16_to_f32(cw.y >> 16), s);
      lut[j * kVqCodes + c] = s * a.sm_scale;
      hist[j * kVqCodes + c] = 0.0f;
    }
  }
  __syncthreads();

  const int lgP = __builtin_ctz(static_cast<unsigned>(a.P));
  const int pmask = a.P - 1;
  const int64_t hb = static_cast<int64_t>(2) * a.P * G;
  const uint8_t* head = a.pool + static_cast<int64_t>(h) * a.num_pages * hb;
  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_pages;
  auto row_of = [&](int t) -> const uint8_t* {
    return head + static_cast<int64_t>(bt[t >> lgP]) * hb + (t & pmask) * G;
  };

  // 2. scores: kTokPerThread tokens per thread, rows loaded before use
  float mloc = -INFINITY;
  for (int t0 = start; t0 < end; t0 += kThreads * kTokPerThread) {
    uint4 w[kTokPerThread][kWords];
#pragma unroll
    for (int u = 0; u < kTokPerThread; ++u) {
      const int t = t0 + u * kThreads + tid;
#pragma unroll
      for (int k = 0; k < kWords; ++k)
        w[u][k] = t < end ? reinterpret_cast<const uint4*>(row_of(t))[k] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kTokPerThread; ++u) {
      const int t = t0 + u * kThreads + tid;
      float s = 0.0f;
#pragma unroll
      for (int k = 0; k < kWords; ++k) {
        const uint32_t ws[4] = {w[u][k].x, w[u][k].y, w[u][k].z, w[u][k].w};
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int j = 16 * k + q;
          s += lut[j * kVqCodes + ((ws[q / 4] >> (8 * (q % 4))) & 0xffu)];
        }
      }
      if (t < end) {
        sc[t - start] = s;
        mloc = fmaxf(mloc, s);
      }
    }
  }
  mloc = wave_max(mloc);
  if ((tid & 63) == 0) red[tid >> 6] = mloc;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) M = fmaxf(M, red[i]);
  __syncthreads();

  // 3. weights into the value-codeword histogram
  float lloc = 0.0f;
  for (int t0 = start; t0 < end; t0 += kThreads * kTokPerThread) {
    uint4 w[kTokPerThread][kWords];
#pragma unroll
    for (int u = 0; u < kTokPerThread; ++u) {
      const int t = t0 + u * kThreads + tid;
#pragma unroll
      for (int k = 0; k < kWords; ++k)
        w[u][k] = t < end ? reinterpret_cast<const uint4*>(row_of(t) + a.P * G)[k] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kTokPerThread; ++u) {
      const int t = t0 + u * kThreads + tid;
      if (t < end) {
        const float p = __expf(sc[t - start] - M);
        lloc += p;
#pragma unroll
        for (int k = 0; k < kWords; ++k) {
          const uint32_t ws[4] = {w[u][k].x, w[u][k].y, w[u][k].z, w[u][k].w};
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int j = 16 * k + q;
            atomicAdd(&hist[j * kVqCodes + ((ws[q / 4] >> (8 * (q % 4))) & 0xffu)], p);
          }
        }
      }
    }
  }
  lloc = wave_sum(lloc);
  if ((tid & 63) == 0) red[tid >> 6] = lloc;
  __syncthreads();
  float Lsum = 0.0f;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) Lsum += red[i];

  // 4. o[4j + e] = sum_c hist[j][c] * value codeword_c[4 loop + e]; each
  //    channel is split over kThreads / D threads (adjacent lanes)
  constexpr int kPer = kThreads / D;             // 2 (D = 128) or 4 (D = 64)
  const int ch = tid / kPer, part_i = tid % kPer;
  const int j = ch / kVqSub, e = ch % kVqSub;
  float acc = 0.0f;
  const uint16_t* cv = a.cb_v + static_cast<int64_t>(j) * kVqCodes * J + kVqSub * a.loop + e;
  for (int c = part_i * (kVqCodes / kPer); c < (part_i + 1) * (kVqCodes / kPer); ++c)
    acc = fmaf(hist[j * kVqCodes + c], f16_to_f32(cv[static_cast<int64_t>(c) * J]), acc);
#pragma unroll
  for (int o = 1; o < kPer; o <<= 1) acc += __shfl_xor(acc, o, 64);
  float* part = a.partials + (pair * a.S + split) * (D + kPartialPad);
  if (part_i == 0) part[kPartialPad + ch] = acc;
  if (tid == 0) {
    part[0] = M;
    part[1] = Lsum;
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
  hipLaunchKernelGGL((vq_split_kernel<D, R>), dim3(a.S, a.H, a.batch), dim3(kThreads), 0, stream, a);
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
