// decode.hip -- plan-driven decode attention over one cell's quantized cache.
//
// Source: "LoopKV: Loop-Aware KV Cache Compression for Serving Looped
// Transformers", abstract (概要): each loop reads the high two bits of every
// 4-bit value and fetches the low two bits only where its own attention
// weights need 4-bit precision; a cell may instead be 2-bit, or reuse the
// final loop's cache of its layer.
//
// Two kernels per call:
//   decode_split_kernel  one wave per (split, head, sequence).  Keys are
//       read at the source's full precision, scores and an online softmax
//       are formed, and values are accumulated from the high plane only (or
//       from both planes when tau = 0).  It writes a partial (max, sum, o)
//       and, when a tau mask is needed, the compacted list of tokens that
//       can still pass the threshold (wave ballot + prefix count).
//   decode_merge_kernel  one wave per (head, sequence).  Log-sum-exp merge of
//       the partials; tokens with p_t >= tau (score >= LSE + ln tau) are
//       flagged with a ballot + prefix count, and only their low-plane rows
//       are fetched to correct the bucket-centre values.
// An unfetched 4-bit value is (4*hi + 3/2)*s + z, so a flagged token adds
// p_t * s * (lo - 3/2).
//
// Arithmetic: a 2-bit field at bit 2i of a byte is masked in place (byte
// value code * 4^i) and converted with one byte-to-float conversion; the
// 4^-i factor is folded into the per-channel multiplier, which keeps the
// products bit-identical to code * multiplier.
#include "device.hpp"
#include "kernels.hpp"

namespace lkv {
namespace {

constexpr int kFlagCap = 512;      // flagged tokens buffered per gather pass

// multiplier of a field at position i of its byte.  "combined" bytes hold a
// 4-bit code (4*hi + lo) built from two planes: positions 0..2 hold
// code * 4^i, position 3 holds code * 16 (see combine()).
template <bool kCombined>
__device__ __forceinline__ constexpr float posf(int i) {
  return i == 0 ? 1.0f : i == 1 ? 0.25f : i == 2 ? 0.0625f : (kCombined ? 0.0625f : 0.015625f);
}

// bytes of the 2-bit fields at position i of each byte of w (value code*4^i)
__device__ __forceinline__ uint32_t field(uint32_t w, int i) {
  return w & (0x03030303u << (2 * i));
}

// 4-bit codes from a high and a low plane word, position i of each byte:
// i < 3: (4*hi + lo) * 4^i;  i == 3: (4*hi + lo) * 16.
__device__ __forceinline__ uint32_t combine(uint32_t hw, uint32_t lw, int i) {
  const uint32_t m = 0x03030303u << (2 * i);
  return i < 3 ? (((hw & m) << 2) | (lw & m)) : ((hw & m) | ((lw & m) >> 2));
}

template <int D, int KIND, int MODE>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
  constexpr int kNJ = D / kGroup;       // value channel groups
  constexpr int kSlots = 64 / kNJ;      // tokens per value step
  constexpr int kWords = D / 16;        // 32-bit words per row
  constexpr int kCPL = D / 32;          // channels per lane in the meta step
  constexpr bool kQ4 = KIND == kKindQ4;
  constexpr bool kSparse = MODE == kModeSparse;
  constexpr bool kDense = MODE == kModeDense;

  __shared__ float qs[D];
  __shared__ float qk[2][D];
  __shared__ float bias_s[2];
  __shared__ float ptile[kTile];
  __shared__ float sc[kSparse ? kMaxSplitLen : 1];

  const int lane = threadIdx.x;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int H = a.H;
  const CellLayout L = a.lay;
  const int T = a.seq_lens[b];
  const int start = split * a.split_len;
  const int end = min(start + a.split_len, T);
  const int64_t pair = static_cast<int64_t>(b) * H + h;
  float* part = a.partials + (pair * a.S + split) * (D + kPartialPad);
  if (start >= end) {
    if (lane == 0) {
      part[0] = -INFINITY;
      part[1] = 0.0f;
      if (kSparse) a.cand_count[pair * a.S + split] = 0;
    }
    for (int d = lane; d < D; d += 64) part[kPartialPad + d] = 0.0f;
    return;
  }

  for (int d = lane; d < D; d += 64) qs[d] = bf16_to_f32(a.q[pair * D + d]) * a.sm_scale;
  __syncthreads();

  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_pages;
  const uint8_t* hbase = a.pool + static_cast<int64_t>(h) * a.num_pages * L.HB;
  const int vj = lane % kNJ, vslot = lane / kNJ;

  float m = -INFINITY, lsum = 0.0f, zs = 0.0f;
  float acc[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) acc[c] = 0.0f;

  for (int t0 = start; t0 < end; t0 += kTile) {
    // --- key metadata of the tile's two key groups -> per-channel multipliers
    {
      const int gsel = lane >> 5;
      const int gtok = t0 + kGroup * gsel;
      const int d0 = (lane & 31) * kCPL;
      float bpart = 0.0f;
      if (gtok < end) {
        const int lp = gtok / L.P, ksl = (gtok % L.P) / kGroup;
        const uint16_t* km = reinterpret_cast<const uint16_t*>(
            hbase + static_cast<int64_t>(bt[lp]) * L.HB + L.off_kmeta + ksl * 4 * D);
#pragma unroll
        for (int c = 0; c < kCPL; ++c) {
          const int d = d0 + c;
          const float s = f16_to_f32(km[d]);
          const float z = f16_to_f32(km[D + d]);
          const float qv = qs[d];
          bpart = fmaf(qv, z, bpart);
          qk[gsel][d] = qv * s * posf<kQ4>(d & 3);
        }
      } else {
#pragma unroll
        for (int c = 0; c < kCPL; ++c) qk[gsel][d0 + c] = 0.0f;
      }
      bpart = half_wave_sum(bpart);
      if ((lane & 31) == 0) bias_s[gsel] = bpart;
    }
    __syncthreads();

    // --- scores: one token per lane, keys at the source's full precision
    const int t = t0 + lane;
    const bool valid = t < end;
    float s_t = -INFINITY;
    if (valid) {
      const int g = lane >> 5;
      const uint8_t* blk = hbase + static_cast<int64_t>(bt[t / L.P]) * L.HB;
      const int r = t % L.P;
      uint32_t hw[kWords], lw[kWords];
      const uint4* ph = reinterpret_cast<const uint4*>(blk + L.off_khi + r * L.row);
#pragma unroll
      for (int v = 0; v < kWords / 4; ++v) {
        const uint4 x = ph[v];
        hw[4 * v] = x.x; hw[4 * v + 1] = x.y; hw[4 * v + 2] = x.z; hw[4 * v + 3] = x.w;
      }
      if (kQ4) {
        const uint4* pl = reinterpret_cast<const uint4*>(blk + L.off_klo + r * L.row);
#pragma unroll
        for (int v = 0; v < kWords / 4; ++v) {
          const uint4 x = pl[v];
          lw[4 * v] = x.x; lw[4 * v + 1] = x.y; lw[4 * v + 2] = x.z; lw[4 * v + 3] = x.w;
        }
      }
      float dot = 0.0f;
#pragma unroll
      for (int k = 0; k < kWords; ++k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t cls = kQ4 ? combine(hw[k], lw[k], i) : field(hw[k], i);
#pragma unroll
          for (int bb = 0; bb < 4; ++bb)
            dot = fmaf(qk[g][16 * k + 4 * bb + i], byte_f(cls, bb), dot);
        }
      }
      s_t = dot + bias_s[g];
    }

    // --- online softmax with a wave-uniform running maximum
    const float tmax = wave_max(s_t);
    if (tmax > m) {
      const float alpha = __expf(m - tmax);
      lsum *= alpha;
      zs *= alpha;
#pragma unroll
      for (int c = 0; c < 32; ++c) acc[c] *= alpha;
      m = tmax;
    }
    const float p = valid ? __expf(s_t - m) : 0.0f;
    lsum += p;
    if (kSparse && valid) sc[t - start] = s_t;
    ptile[lane] = p;
    __syncthreads();

    // --- values: lane = (token slot, 32-channel group); high plane only
    //     (both planes in dense mode)
#pragma unroll
    for (int sub = 0; sub < kTile; sub += kSlots) {
      const int tt = t0 + sub + vslot;
      if (tt < end) {
        const float pp = ptile[sub + vslot];
        const uint8_t* blk = hbase + static_cast<int64_t>(bt[tt / L.P]) * L.HB;
        const int r = tt % L.P;
        const uint32_t meta = reinterpret_cast<const uint32_t*>(blk + L.off_vmeta)[r * kNJ + vj];
        const float vs = f16_to_f32(meta & 0xffffu), vz = f16_to_f32(meta >> 16);
        const uint2 hv = *reinterpret_cast<const uint2*>(blk + L.off_vhi + r * L.row + 8 * vj);
        const uint32_t hw2[2] = {hv.x, hv.y};
        uint32_t lw2[2] = {0u, 0u};
        float w;
        if (kQ4 && kDense) {
          const uint2 lv = *reinterpret_cast<const uint2*>(blk + L.off_vlo + r * L.row + 8 * vj);
          lw2[0] = lv.x;
          lw2[1] = lv.y;
          w = pp * vs;
          zs = fmaf(pp, vz, zs);
        } else if (kQ4) {
          w = pp * vs * 4.0f;                       // high plane weight 4*s
          zs = fmaf(pp, fmaf(1.5f, vs, vz), zs);    // bucket centre + zero
        } else {
          w = pp * vs;
          zs = fmaf(pp, vz, zs);
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t cls = (kQ4 && kDense) ? combine(hw2[e], lw2[e], i) : field(hw2[e], i);
            const float wi = w * ((kQ4 && kDense) ? posf<true>(i) : posf<false>(i));
#pragma unroll
            for (int bb = 0; bb < 4; ++bb)
              acc[16 * e + 4 * bb + i] = fmaf(wi, byte_f(cls, bb), acc[16 * e + 4 * bb + i]);
          }
        }
      }
    }
    __syncthreads();
  }

  // --- partial: sum the token slots of each channel group
#pragma unroll
  for (int o = kNJ; o < 64; o <<= 1) {
#pragma unroll
    for (int c = 0; c < 32; ++c) acc[c] += __shfl_xor(acc[c], o, 64);
    zs += __shfl_xor(zs, o, 64);
  }
  lsum = wave_sum(lsum);
  if (lane < kNJ) {
#pragma unroll
    for (int c = 0; c < 32; ++c) part[kPartialPad + kGroup * lane + c] = acc[c] + zs;
  }
  if (lane == 0) {
    part[0] = m;
    part[1] = lsum;
  }

  // --- candidates: tokens that pass tau against this split's own LSE.  The
  //     split's LSE is <= the global one, so no true flag is dropped; the
  //     merge kernel takes the final decision.  A small margin covers
  //     rounding of this local test.
  if (kSparse) {
    const float theta = m + logf(lsum) + a.log_tau - 1e-3f;
    int2* cl = a.cand + (pair * a.S + split) * a.split_len;
    const int n = end - start;
    int count = 0;
    for (int base = 0; base < n; base += 64) {
      const int idx = base + lane;
      const float v = idx < n ? sc[idx] : -INFINITY;
      const bool f = v >= theta;
      const uint64_t bal = __ballot(f);
      const int pos = __popcll(bal & ((1ull << lane) - 1ull));
      if (f) cl[count + pos] = make_int2(start + idx, __float_as_int(v));
      count += __popcll(bal);
    }
    if (lane == 0) a.cand_count[pair * a.S + split] = count;
  }
}

template <int D, int KIND, int MODE>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  constexpr int kNJ = D / kGroup;
  constexpr int kSlots = 64 / kNJ;
  constexpr bool kSparse = MODE == kModeSparse;
  constexpr bool kDense = MODE == kModeDense;

  __shared__ float ew[kMaxSplits];
  __shared__ float o_s[D];
  __shared__ int fl_t[kSparse ? kFlagCap : 1];
  __shared__ float fl_p[kSparse ? kFlagCap : 1];

  const int lane = threadIdx.x;
  const int h = blockIdx.x, b = blockIdx.y;
  const int H = a.H;
  const CellLayout L = a.lay;
  const int T = a.seq_lens[b];
  const int64_t pair = static_cast<int64_t>(b) * H + h;
  float* outp = a.out + pair * D;
  uint32_t* mrow = a.mask_bits ? a.mask_bits + pair * a.mask_words : nullptr;

  if (mrow) {
    for (int w = lane; w < a.mask_words; w += 64) {
      uint32_t bits = 0u;
      if (kDense) {
        const int lo = 32 * w;
        bits = T >= lo + 32 ? 0xffffffffu : (T > lo ? ((1u << (T - lo)) - 1u) : 0u);
      }
      mrow[w] = bits;
    }
    __threadfence();
  }
  if (T <= 0) {
    for (int d = lane; d < D; d += 64) outp[d] = 0.0f;
    return;
  }

  // lengths above max_seq_len break the caller's contract; never read past S
  const int S_used = min((T + a.split_len - 1) / a.split_len, a.S);
  const float* parts = a.partials + pair * a.S * (D + kPartialPad);
  constexpr int kRec = D + kPartialPad;

  float M = -INFINITY;
  for (int i = lane; i < S_used; i += 64) M = fmaxf(M, parts[i * kRec]);
  M = wave_max(M);
  float lsum = 0.0f;
  for (int i = lane; i < S_used; i += 64) {
    const float e = __expf(parts[i * kRec] - M);
    ew[i] = e;
    lsum = fmaf(e, parts[i * kRec + 1], lsum);
  }
  lsum = wave_sum(lsum);
  __syncthreads();
  const float inv = 1.0f / lsum;
  const float lse = M + logf(lsum);
  for (int d = lane; d < D; d += 64) {
    float o = 0.0f;
    for (int i = 0; i < S_used; ++i) o = fmaf(ew[i], parts[i * kRec + kPartialPad + d], o);
    o_s[d] = o * inv;
  }

  unsigned long long flagged = 0ull;
  if (kSparse) {
    const float theta = lse + a.log_tau;
    const int vj = lane % kNJ, vslot = lane / kNJ;
    float corr[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) corr[c] = 0.0f;
    float cs = 0.0f;
    int nf = 0;

    auto gather = [&](int count) {
      for (int base = 0; base < count; base += kSlots) {
        const int idx = base + vslot;
        if (idx < count) {
          const int t = fl_t[idx];
          const float pp = fl_p[idx];
          const uint8_t* blk = a.pool + (static_cast<int64_t>(h) * a.num_pages +
                                         a.block_tables[static_cast<int64_t>(b) * a.max_pages + t / L.P]) * L.HB;
          const int r = t % L.P;
          const uint32_t meta = reinterpret_cast<const uint32_t*>(blk + L.off_vmeta)[r * kNJ + vj];
          const float vs = f16_to_f32(meta & 0xffffu);
          const uint2 lv = *reinterpret_cast<const uint2*>(blk + L.off_vlo + r * L.row + 8 * vj);
          const uint32_t lw2[2] = {lv.x, lv.y};
          const float w = pp * vs;
          cs += w;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t cls = field(lw2[e], i);
              const float wi = w * posf<false>(i);
#pragma unroll
              for (int bb = 0; bb < 4; ++bb)
                corr[16 * e + 4 * bb + i] = fmaf(wi, byte_f(cls, bb), corr[16 * e + 4 * bb + i]);
            }
          }
        }
      }
    };

    for (int i = 0; i < S_used; ++i) {
      const int cnt = a.cand_count[pair * a.S + i];
      const int2* cl = a.cand + (pair * a.S + i) * a.split_len;
      for (int base = 0; base < cnt; base += 64) {
        const int k = base + lane;
        int2 c = make_int2(0, 0);
        if (k < cnt) c = cl[k];
        const float s = __int_as_float(c.y);
        const bool f = (k < cnt) && (s >= theta);
        const uint64_t bal = __ballot(f);
        const int pos = __popcll(bal & ((1ull << lane) - 1ull));
        if (f) {
          fl_t[nf + pos] = c.x;
          fl_p[nf + pos] = expf(s - lse);
          if (mrow && (c.x >> 5) < a.mask_words) atomicOr(&mrow[c.x >> 5], 1u << (c.x & 31));
        }
        nf += __popcll(bal);
        if (nf > kFlagCap - 64) {
          __syncthreads();
          gather(nf);
          flagged += nf;
          nf = 0;
          __syncthreads();
        }
      }
    }
    __syncthreads();
    gather(nf);
    flagged += nf;

#pragma unroll
    for (int o = kNJ; o < 64; o <<= 1) {
#pragma unroll
      for (int c = 0; c < 32; ++c) corr[c] += __shfl_xor(corr[c], o, 64);
      cs += __shfl_xor(cs, o, 64);
    }
    __syncthreads();
    if (lane < kNJ) {
#pragma unroll
      for (int c = 0; c < 32; ++c) o_s[kGroup * lane + c] += corr[c] - 1.5f * cs;
    }
  } else if (kDense) {
    flagged = static_cast<unsigned long long>(T);
  }
  if (a.counters && lane == 0 && (kSparse || kDense)) {
    atomicAdd(&a.counters[0], flagged);
    atomicAdd(&a.counters[1], flagged * static_cast<unsigned long long>(L.row));
  }
  __syncthreads();
  for (int d = lane; d < D; d += 64) outp[d] = o_s[d];
}

template <int D, int KIND, int MODE>
hipError_t launch_typed(const DecodeArgs& a, int batch, hipStream_t stream) {
  prof_mark(kClassSplit, 0, stream);
  hipLaunchKernelGGL((decode_split_kernel<D, KIND, MODE>), dim3(a.S, a.H, batch), dim3(64), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_mark(kClassSplit, 1, stream);
  prof_mark(kClassMerge, 0, stream);
  hipLaunchKernelGGL((decode_merge_kernel<D, KIND, MODE>), dim3(a.H, batch), dim3(64), 0, stream,
                     a);
  e = hipGetLastError();
  prof_mark(kClassMerge, 1, stream);
  return e;
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, int batch, int mode, hipStream_t stream) {
  if (a.lay.kind == kKindQ2) return launch_typed<D, kKindQ2, kModePlain>(a, batch, stream);
  if (mode == kModeSparse) return launch_typed<D, kKindQ4, kModeSparse>(a, batch, stream);
  if (mode == kModeDense) return launch_typed<D, kKindQ4, kModeDense>(a, batch, stream);
  return launch_typed<D, kKindQ4, kModePlain>(a, batch, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int batch, int mode, hipStream_t stream) {
  return a.lay.D == 128 ? launch_d<128>(a, batch, mode, stream) : launch_d<64>(a, batch, mode, stream);
}

}  // namespace lkv
