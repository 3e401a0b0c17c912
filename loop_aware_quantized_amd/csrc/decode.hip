// decode.hip -- plan-driven decode attention over one cell's quantized cache.
//
// Source: "LoopKV: Loop-Aware KV Cache Compression for Serving Looped
// Transformers", abstract (概要): a decoding loop always uses the upper two
// bits of a 4-bit value and loads the lower two only for tokens whose
// weight under that loop's own query is large enough to need them; other
// cells hold 2-bit codes or borrow the last loop's cache of their layer.
//
// Two kernels per call:
//   decode_split_kernel  one wave per (split, head, sequence).  Keys are
//       read at the source's full precision, scores and an online softmax
//       are formed, and values are accumulated from the high plane only (or
//       from both planes when tau = 0).  It writes a partial (max, sum, o)
//       and, when a tau mask is needed, the compacted list of tokens that
//       can still pass the threshold (wave ballot + prefix count).  The
//       first split of a (sequence, head) also clears its mask row.
//   decode_merge_kernel  one wave per (head, sequence).  Log-sum-exp merge of
//       the partials; tokens with p_t >= tau (score >= LSE + ln tau) are
//       flagged with a ballot + prefix count, and only their low-plane rows
//       are fetched to correct the bucket-centre values.
// The kernel boundary orders the two: a merge inside the split kernel (last
// split to arrive) would need a device-scope release per wave, which on
// this chip writes back the XCD's L2 and measured several times slower.
// An unfetched 4-bit value is (4*hi + 3/2)*s + z, so a flagged token adds
// p_t * s * (lo - 3/2).
//
// Arithmetic: key fields are masked in place inside 16-bit halves, where
// they read as fp16 subnormals code * 2^k * 2^-24; a mixed-precision FMA
// widens them as it multiplies, and the 2^24 * 2^-k is folded into the
// per-channel multiplier, so every product is exactly code * multiplier.
// Value fields take the same form in packed fp16 dot products (two tokens
// per instruction); the tau = 0 path converts bytes through fp8.
#include "device.hpp"
#include "kernels.hpp"

namespace lkv {
namespace {

constexpr int kFlagCap = 512;      // flagged tokens buffered per gather pass
constexpr int kCandCap = 256;      // candidates buffered in LDS per split wave
// cache-policy operand of the pool's buffer loads: bit 1 = non-temporal
constexpr int kStreamLoad = 2;
// largest weight exponent: 2^(14 - floor(log2 s)) for the smallest fp16
// scale s = 2^-24 is 2^38
constexpr int kMaxWeightExp = 40;
constexpr float kLn2 = 0.693147180559945309f;

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

// Converts the four bytes of w, each holding an integer n < 16, to floats.
// An fp8 (e4m3) byte below 16 is a subnormal or lies in the first normal
// binade, whose spacing is the same, so it converts to exactly n * unit with
// unit a power of two fixed by the format (read back at run time).
__device__ __forceinline__ void cvt_bytes(uint32_t w, float* f) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  f[0] = lo[0]; f[1] = lo[1]; f[2] = hi[0]; f[3] = hi[1];
}

// Unpacks a high-plane word and a low-plane word into 16 four-bit codes
// 4*hi + lo as floats, in the same position order p = 4i + b.
__device__ __forceinline__ void unpack_combined(uint32_t h, uint32_t l, float* f) {
  // even fields (i = 0, 2) as nibbles: lo bits stay, hi bits move up by 2
  const uint32_t e = ((h << 2) & 0xCCCCCCCCu) | (l & 0x33333333u);
  // odd fields (i = 1, 3): hi bits stay, lo bits move down by 2
  const uint32_t o = (h & 0xCCCCCCCCu) | ((l >> 2) & 0x33333333u);
  cvt_bytes(e & 0x0F0F0F0Fu, f);
  cvt_bytes(o & 0x0F0F0F0Fu, f + 4);
  cvt_bytes((e >> 4) & 0x0F0F0F0Fu, f + 8);
  cvt_bytes((o >> 4) & 0x0F0F0F0Fu, f + 12);
}

// Key words as pairs of fp16 halves.  A 2-bit field (or a 4-bit code)
// masked in place inside a 16-bit half is an fp16 subnormal
// code * 2^k * 2^-24 (exact), which a mixed-precision FMA widens to fp32
// as it multiplies; the 2^24 * 2^-k lands in the channel's multiplier.
// pr[2i] holds field i of bytes 0 and 2, pr[2i + 1] field i of bytes 1
// and 3 (read from w >> 6, so they arrive times 4).
__device__ __forceinline__ void key_pairs_plain(uint32_t w, uint32_t* pr) {
  const uint32_t u = w >> 6;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pr[2 * i] = w & (0x00030003u << (2 * i));
    pr[2 * i + 1] = u & (0x000C000Cu << (2 * i));
  }
}

// The same for 4-bit codes 4*hi + lo built from a high-plane and a
// low-plane word: even fields as the low nibbles of e, odd ones of o; the
// nibble of fields 2 and 3 arrives times 16.
__device__ __forceinline__ void key_pairs_combined(uint32_t h, uint32_t l, uint32_t* pr) {
  const uint32_t e = ((h << 2) & 0xCCCCCCCCu) | (l & 0x33333333u);
  const uint32_t o = (h & 0xCCCCCCCCu) | ((l >> 2) & 0x33333333u);
  const uint32_t e6 = e >> 6, o6 = o >> 6;
  pr[0] = e & 0x000F000Fu; pr[1] = e6 & 0x003C003Cu;   // field 0
  pr[2] = o & 0x000F000Fu; pr[3] = o6 & 0x003C003Cu;   // field 1
  pr[4] = e & 0x00F000F0u; pr[5] = e6 & 0x03C003C0u;   // field 2
  pr[6] = o & 0x00F000F0u; pr[7] = o6 & 0x03C003C0u;   // field 3
}

__device__ __forceinline__ float half_lo(uint32_t x) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(x)));
}
__device__ __forceinline__ float half_hi(uint32_t x) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(x >> 16)));
}

// channel (within a 16-channel word) of position p = 4i + b (field i of
// byte b), and back
__host__ __device__ constexpr int pos_channel(int p) { return 4 * (p % 4) + p / 4; }
__host__ __device__ constexpr int channel_pos(int m) { return 4 * (m % 4) + m / 4; }
// multiplier factor of key position p: undoes the 2^-24 of the subnormal
// and the 2^k at which the field sits in its half
template <bool kCombined>
__device__ __forceinline__ constexpr float key_factor(int p) {
  const int i = p / 4, odd_byte = p & 1;
  return kCombined ? 16777216.0f / static_cast<float>(1 << (4 * (i / 2) + 2 * odd_byte))
                   : 16777216.0f / static_cast<float>(1 << (2 * (i + odd_byte)));
}
// value position p = 4i + b accumulated as fp16 subnormals code * 4^i * 2^-24
__device__ __forceinline__ constexpr float dot2_factor(int p) {
  return 16777216.0f / static_cast<float>(1 << (2 * (p / 4)));
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Everything one 64-token tile reads from HBM, held in registers so the next
// tile's loads are in flight while the current tile computes.
template <int D, bool kQ4, bool kDense>
struct TileData {
  static constexpr int kNJ = D / kGroup;
  static constexpr int kSubs = kTile / (64 / kNJ);
  uint4 kh[D / 64];                 // this lane's token: key row (high plane)
  uint4 kl[kQ4 ? D / 64 : 1];       // key row, low plane
  uint2 vh[kSubs];                  // value rows: 32 channels of one token each
  uint2 vl[kDense ? kSubs : 1];
  uint32_t vm[kSubs];               // value (scale, zero) of that token/group
  uint32_t ks[D / 64], kz[D / 64];  // key-group scale / zero of this lane's channels
};

__device__ __forceinline__ int range_start(const DecodeArgs& a, int w) {
  return w < a.main_waves ? w * a.tiles_per_wave
                          : a.main_waves * a.tiles_per_wave + (w - a.main_waves) * a.tail_tiles;
}
// Ranges continue past the grid with tail_tiles each (a length-sum hint
// below the real sum leaves tiles there); the grid's last wave takes them
// in turn, one record per range as for any other wave.
__device__ __forceinline__ int wave_of(const DecodeArgs& a, int t) {
  const int m = a.main_waves * a.tiles_per_wave;
  return t < m ? t / a.tiles_per_wave : a.main_waves + (t - m) / a.tail_tiles;
}
// A sequence's length in the streamed layout, capped at the caller's
// maximum (cand_stride is that maximum rounded up to a tile) so that a
// length breaking the contract still reads and writes in bounds.
__device__ __forceinline__ int streamed_len(const DecodeArgs& a, int b) {
  return min(max(a.seq_lens[b], 0), a.cand_stride);
}

// One wave per (head, sequence): log-sum-exp merge of the S_used partials,
// then (sparse mode) the exact test p_t >= tau over the candidate lists,
// the mask bits and the low-plane correction of the flagged tokens.  The
// kernel is a chain of dependent reads, so each step issues its reads for
// many splits / candidates / tokens at once.
template <int D, int KIND, int MODE>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  constexpr int kNJ = D / kGroup;
  constexpr int kSlots = 64 / kNJ;
  constexpr int kRec = D + kPartialPad;
  constexpr int kCPL = D / 64;           // output channels per lane
  constexpr int kPass = 4;               // candidates per lane per scan pass
  constexpr int kFirst = 16;             // records requested with the length
  constexpr bool kSparse = MODE == kModeSparse;
  constexpr bool kDense = MODE == kModeDense;
  static_assert(kFlagCap >= 2 * 64 * kPass, "flag buffer must hold two scan passes");

  __shared__ float o_s[D];
  __shared__ int fl_t[kSparse ? kFlagCap : 1];        // flagged tokens awaiting their low rows
  __shared__ float fl_p[kSparse ? kFlagCap : 1];      // their weights p_t
  __shared__ uint32_t fl_pg[kSparse ? kFlagCap : 1];  // their page's offset in the head region
  __shared__ int pre[kSparse ? 64 : 1];               // inclusive prefix of list lengths

  const int lane = threadIdx.x;
  const int h = blockIdx.x, b = blockIdx.y;
  const CellLayout L = a.lay;
  const int64_t pair = static_cast<int64_t>(b) * a.H + h;
  float* outp = a.out + pair * D;
  const float* parts = a.partials + pair * a.S * kRec;

  // --- log-sum-exp merge: lanes over splits for (max, sum); lanes over
  //     channels for o, each split's weight broadcast from its lane.  The
  //     (max, sum) of the first 64 split slots, the first kFirst records and
  //     (sparse) the candidate counts are requested together with the
  //     length, so with up to kFirst splits the merge waits for memory once.
  //     Slots past the sequence's splits hold stale values; they are masked
  //     once the length is known.
  float2 ml_raw = make_float2(-INFINITY, 0.0f);
  if (lane < a.S) ml_raw = *reinterpret_cast<const float2*>(parts + lane * kRec);
  const int cnt_raw = (kSparse && lane < a.S) ? a.cand_count[pair * a.S + lane] : 0;
  // records requested before the length arrives
  const int n_first = min(kFirst, a.S);
  float v0[kFirst][kCPL];
#pragma unroll
  for (int u = 0; u < kFirst; ++u) {
    const float* rec = parts + (u < a.S ? u : 0) * kRec + kPartialPad;
#pragma unroll
    for (int c = 0; c < kCPL; ++c) v0[u][c] = u < n_first ? rec[lane + 64 * c] : 0.0f;
  }
  // streamed layout: tiles (all heads) of the sequences before this one
  int tiles_before = 0;
  if (a.streamed) {
#pragma unroll
    for (int k = 0; k < kMaxStreamedBatch / 64; ++k) {
      const int bb = lane + 64 * k;
      tiles_before += bb < b ? a.H * ((streamed_len(a, bb) + kTile - 1) / kTile) : 0;
    }
  }
  const int T = a.streamed ? streamed_len(a, b) : a.seq_lens[b];
  uint32_t* mrow = a.mask_bits ? a.mask_bits + pair * a.mask_words : nullptr;
  if (T <= 0) {
    for (int d = lane; d < D; d += 64) outp[d] = 0.0f;
    // no split of an empty pair runs in a streamed layout: its row is cleared here
    if (mrow)
      for (int w = lane; w < a.mask_words; w += 64) mrow[w] = 0u;
    return;
  }
  // Records of the pair and the first token of each.  Uniform: record r is
  // split r.  Streamed: the pair's tiles start at tile0 of the end-to-end
  // order, and record r is the part of range (wave_of(tile0) + r) in it.
  int tile0 = 0, w0 = 0, S_used;
  if (a.streamed) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) tiles_before += __shfl_xor(tiles_before, o, 64);
    const int nb = (T + kTile - 1) / kTile;
    tile0 = tiles_before + h * nb;
    w0 = wave_of(a, tile0);
    S_used = min(wave_of(a, tile0 + nb - 1) - w0 + 1, a.S);
  } else {
    // lengths above max_seq_len break the caller's contract; never read past S
    S_used = min((T + a.split_len - 1) / a.split_len, a.S);
  }
  auto rec_start = [&](int r) -> int {
    return a.streamed ? max(0, range_start(a, w0 + r) - tile0) * kTile : r * a.split_len;
  };
  // the row was cleared by the split kernel (the split holding token 0)
  const float m_l = lane < S_used ? ml_raw.x : -INFINITY;
  const float l_l = lane < S_used ? ml_raw.y : 0.0f;
  const int cnt0 = lane < S_used ? cnt_raw : 0;
  float M = m_l;
  for (int i = lane + 64; i < S_used; i += 64) M = fmaxf(M, parts[i * kRec]);
  M = dpp_wave_max(M);
  const float e0 = lane < S_used ? __expf(m_l - M) : 0.0f;   // weight of split `lane`
  float lsum = e0 * l_l;
  for (int i = lane + 64; i < S_used; i += 64) lsum = fmaf(__expf(parts[i * kRec] - M), parts[i * kRec + 1], lsum);
  lsum = dpp_wave_sum(lsum);
  const float inv = 1.0f / lsum;
  const float lse = M + logf(lsum);
  {
    float o[kCPL];
#pragma unroll
    for (int c = 0; c < kCPL; ++c) o[c] = 0.0f;
#pragma unroll
    for (int u = 0; u < kFirst; ++u) {
      const float e = lane_f(e0, u);
#pragma unroll
      for (int c = 0; c < kCPL; ++c)
        o[c] = u < S_used && u < n_first ? fmaf(e, v0[u][c], o[c]) : o[c];   // stale past S_used
    }
    for (int i0 = 0; i0 < S_used; i0 += 64) {
      const int n = min(64, S_used - i0);
      const float e_l = i0 == 0 ? e0 : (lane < n ? __expf(parts[(i0 + lane) * kRec] - M) : 0.0f);
      // sixteen records per step, all loads issued before the first use
      for (int j = i0 == 0 ? n_first : 0; j < n; j += 16) {
        float v[16][kCPL];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float* rec = parts + (i0 + j + u) * kRec + kPartialPad;
#pragma unroll
          for (int c = 0; c < kCPL; ++c) v[u][c] = (j + u < n) ? rec[lane + 64 * c] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float e = lane_f(e_l, (j + u) & 63);   // 0 past n
#pragma unroll
          for (int c = 0; c < kCPL; ++c) o[c] = fmaf(e, v[u][c], o[c]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < kCPL; ++c) o_s[lane + 64 * c] = o[c] * inv;
  }

  unsigned long long flagged = 0ull;
  if (kSparse) {
    const float theta = lse + a.log_tau;
    const int lgP = __builtin_ctz(static_cast<unsigned>(L.P));
    const int pmask = L.P - 1;
    const uint8_t* head = a.pool + static_cast<int64_t>(h) * a.num_pages * L.HB;
    const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_pages;
    const int vj = lane % kNJ, vslot = lane / kNJ;
    float corr[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) corr[c] = 0.0f;
    float cs = 0.0f;
    int nf = 0;

    // low-plane rows of the buffered flagged tokens: their page offsets
    // first (all table reads in flight), then lane = (token slot, 32-channel
    // group) accumulates p_t * s * lo
    auto gather = [&](int count) {
      __syncthreads();
      for (int idx = lane; idx < count; idx += 64)
        fl_pg[idx] = static_cast<uint32_t>(bt[fl_t[idx] >> lgP]) * static_cast<uint32_t>(L.HB);
      __syncthreads();
      for (int base = 0; base < count; base += kSlots) {
        const int idx = base + vslot;
        if (idx < count) {
          const int r = fl_t[idx] & pmask;
          const float pp = fl_p[idx];
          const uint8_t* blk = head + fl_pg[idx];
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
      __syncthreads();
    };

    // The lists of up to 64 splits are scanned as one flat sequence, kPass
    // entries per lane per pass: entry k finds its split by a branch-free
    // binary search over the inclusive prefix of the list lengths (six LDS
    // steps, the kPass searches interleaved).
    for (int i0 = 0; i0 < S_used; i0 += 64) {
      const int ns = min(64, S_used - i0);
      const int cnt = i0 == 0 ? cnt0 : (lane < ns ? a.cand_count[pair * a.S + i0 + lane] : 0);
      const int incl = wave_incl_scan(cnt);
      const int total = __builtin_amdgcn_readlane(incl, 63);
      pre[lane] = incl;
      __syncthreads();
      for (int base = 0; base < total; base += 64 * kPass) {
        if (nf > kFlagCap - 64 * kPass) {
          gather(nf);
          flagged += nf;
          nf = 0;
        }
        // split of entry k: the number of lists that end at or before k
        // (pre[] of lanes past ns holds the total, which exceeds any k)
        int sp[kPass];
#pragma unroll
        for (int u = 0; u < kPass; ++u) sp[u] = 0;
#pragma unroll
        for (int step = 32; step > 0; step >>= 1) {
#pragma unroll
          for (int u = 0; u < kPass; ++u) {
            const int k = base + 64 * u + lane;
            sp[u] += pre[sp[u] + step - 1] <= k ? step : 0;
          }
        }
        int2 c[kPass];
#pragma unroll
        for (int u = 0; u < kPass; ++u) {
          const int k = base + 64 * u + lane;
          c[u] = make_int2(0, 0);
          if (k < total) {
            const int before = sp[u] ? pre[sp[u] - 1] : 0;
            c[u] = a.cand[pair * a.cand_stride + rec_start(i0 + sp[u]) + (k - before)];
          }
        }
#pragma unroll
        for (int u = 0; u < kPass; ++u) {
          const int k = base + 64 * u + lane;
          const float sc = __int_as_float(c[u].y);
          const bool f = (k < total) && (sc >= theta);
          const uint64_t bal = __ballot(f);
          if (f) {
            const int pos = nf + __popcll(bal & ((1ull << lane) - 1ull));
            fl_t[pos] = c[u].x;
            fl_p[pos] = expf(sc - lse);
            if (mrow && (c[u].x >> 5) < a.mask_words) atomicOr(&mrow[c[u].x >> 5], 1u << (c[u].x & 31));
          }
          nf += __popcll(bal);
        }
      }
      __syncthreads();
    }
    gather(nf);
    flagged += nf;

    // sum the token slots of each channel group (lanes of equal lane % kNJ)
#pragma unroll
    for (int c = 0; c < 32; ++c) corr[c] = strided_sum<kNJ>(corr[c]);
    cs = strided_sum<kNJ>(cs);
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

// One split of one (sequence, head): tokens [start, end) of sequence b
// (length T), head h; its partial record is number rec of the pair, and
// `first` marks the split holding the pair's first token (which owns the
// pair's mask row).  kStreamed: called by the streamed-layout kernel.
template <int D, int KIND, int MODE, bool kStreamed>
__device__ __forceinline__ void split_segment(const DecodeArgs& a, const int b, const int h, const int T,
                                              const int start, const int end, const int rec, const bool first) {
  constexpr int kNJ = D / kGroup;       // value channel groups
  constexpr int kSlots = 64 / kNJ;      // tokens per value step
  constexpr int kSubs = kTile / kSlots; // value steps per tile
  constexpr int kWords = D / 16;        // 32-bit words per row
  constexpr int kCPL = D / 32;          // channels per lane in the meta step
  constexpr bool kQ4 = KIND == kKindQ4;
  constexpr bool kSparse = MODE == kModeSparse;
  constexpr bool kDense = MODE == kModeDense;
  constexpr bool kKeyComb = kQ4;            // keys: 4-bit codes from two planes
  constexpr bool kValComb = kQ4 && kDense;  // values: both planes only when tau = 0
  using Tile = TileData<D, kQ4, kDense>;

  __shared__ float qs[D];
  __shared__ float qk[2][D];                 // per-channel key multipliers, position order
  __shared__ float ptile[kTile];
  // byte offset of the split's i-th page inside this head's pool region
  // (+4: the prefetch of the tile after the last one may index past np)
  __shared__ uint32_t pgoff[kMaxSplitLen / 16 + 4];
  __shared__ int2 cbuf[kSparse ? kCandCap : 1];   // candidate (token, score bits)

  const int lane = threadIdx.x;
  const int H = a.H;
  const CellLayout L = a.lay;
  const int64_t pair = static_cast<int64_t>(b) * H + h;
  float* part = a.partials + (pair * a.S + rec) * (D + kPartialPad);
  // page size is a power of two; splits and tiles start on page boundaries
  const int lgP = __builtin_ctz(static_cast<unsigned>(L.P));
  const int pmask = L.P - 1;
  // The block-table slice of the split's whole span (clamped to the row)
  // and the query are requested before the length is known, so that their
  // reads overlap the length's; entries past the sequence are dropped below.
  constexpr int kPgSlots = kMaxSplitLen / 16 + 4;
  constexpr int kPgPerLane = (kPgSlots + 63) / 64;
  uint32_t pg_raw[kPgPerLane];
  {
    const int first = start >> lgP;
    const int span = min((a.split_len + pmask) >> lgP, a.max_pages - first);
    const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_pages + first;
#pragma unroll
    for (int k = 0; k < kPgPerLane; ++k) {
      const int i = lane + 64 * k;
      pg_raw[k] = i < span ? static_cast<uint32_t>(bt[i]) : 0u;
    }
  }
  float q_raw[D / 64];
#pragma unroll
  for (int c = 0; c < D / 64; ++c) q_raw[c] = bf16_to_f32(a.q[pair * D + lane + 64 * c]);

  if (first && a.mask_bits) {
    // the first split owns the pair's mask row: cleared here (all ones up to
    // T for tau = 0); the merge kernel, launched after, sets the flag bits
    uint32_t* mrow = a.mask_bits + pair * a.mask_words;
    for (int w = lane; w < a.mask_words; w += 64) {
      uint32_t bits = 0u;
      if (kDense) {
        const int lo = 32 * w;
        bits = T >= lo + 32 ? 0xffffffffu : (T > lo ? ((1u << (T - lo)) - 1u) : 0u);
      }
      mrow[w] = bits;
    }
  }
  if (start >= end) {         // splits past the end take no part in the merge
    // one split per pair and no merge launch: the empty pair's output is zero
    if (!kSparse && a.direct_out && rec == 0)
      for (int d = lane; d < D; d += 64) a.out[pair * D + d] = 0.0f;
    return;
  }

  {
    const int np = ((end - start) + pmask) >> lgP;   // <= span: end <= T <= max_pages * P
#pragma unroll
    for (int k = 0; k < kPgPerLane; ++k) {
      const int i = lane + 64 * k;
      if (i < kPgSlots) pgoff[i] = i < np ? pg_raw[k] * static_cast<uint32_t>(L.HB) : 0u;
    }
  }
#pragma unroll
  for (int c = 0; c < D / 64; ++c) qs[lane + 64 * c] = q_raw[c] * a.sm_scale;
  __syncthreads();

  // this head's pool region as a raw buffer: 32-bit offsets, and loads past
  // the region return zero instead of faulting.  A region of no records
  // turns the loads issued for a split's last tile (see the tile loop) into
  // ones that return zeros without a memory request.
  uint8_t* const region_base = const_cast<uint8_t*>(a.pool + static_cast<int64_t>(h) * a.num_pages * L.HB);
  const int region_bytes = static_cast<int>(static_cast<uint32_t>(a.num_pages * L.HB));
  auto region = [&](bool live) {
    return __builtin_amdgcn_make_buffer_rsrc(region_base, static_cast<short>(0), live ? region_bytes : 0,
                                             0x00020000);
  };
  const int vj = lane % kNJ, vslot = lane / kNJ;
  const int gsel = lane >> 5;
  const int d0 = (lane & 31) * kCPL;
  const float unit = __builtin_amdgcn_cvt_pk_f32_fp8(1, false)[0];
  const float inv_unit = 1.0f / unit;
  // lane-constant parts of the load offsets
  const uint32_t lane_krow = static_cast<uint32_t>((lane & pmask) * (D / 4));
  const int lane_kpage = lane >> lgP;
  const uint32_t lane_vrow = static_cast<uint32_t>(vslot * (D / 4) + 8 * vj);
  const uint32_t lane_vmeta = static_cast<uint32_t>((vslot * kNJ + vj) * 4);
  const int lane_mpage = (kGroup * gsel) >> lgP;
  const uint32_t lane_kmeta = static_cast<uint32_t>(L.off_kmeta + (((kGroup * gsel) & pmask) / kGroup) * 4 * D + 2 * d0);

  // The cache is streamed: every byte is read once per launch.  Loads carry
  // the non-temporal hint, which raises this chip's streaming-read rate by
  // about 12% (6.1 -> 6.9 TB/s on an 805 MB read).
  // Issue every load of the tile starting at t0 (live: into the head's
  // region; else the same instructions over an empty region).  Rows past
  // the split's end read whatever their (possibly unmapped) page offsets
  // point to inside the head's region; the buffer bounds keep that safe and
  // the results are masked out.
  auto fetch = [&](Tile& td, int t0, bool live) {
    const auto rsrc = region(live);
    auto ld128 = [&](uint32_t voff, uint32_t soff) -> uint4 {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, soff, kStreamLoad);
      return make_uint4(v[0], v[1], v[2], v[3]);
    };
    auto ld64 = [&](uint32_t voff, uint32_t soff) -> uint2 {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(rsrc, voff, soff, kStreamLoad);
      return make_uint2(v[0], v[1]);
    };
    auto ld32 = [&](uint32_t voff, uint32_t soff) -> uint32_t {
      return __builtin_amdgcn_raw_buffer_load_b32(rsrc, voff, soff, kStreamLoad);
    };
    const int tp0 = (t0 - start) >> lgP;
    {
      const uint32_t ro = pgoff[tp0 + lane_kpage] + lane_krow;
#pragma unroll
      for (int v = 0; v < D / 64; ++v) td.kh[v] = ld128(ro, L.off_khi + 16 * v);
      if (kQ4) {
#pragma unroll
        for (int v = 0; v < D / 64; ++v) td.kl[v] = ld128(ro, L.off_klo + 16 * v);
      }
    }
#pragma unroll
    for (int sub = 0; sub < kSubs; ++sub) {
      const int first = sub * kSlots;
      if (kSlots <= 16) {
        // a value step's 16 tokens share one page (pages hold >= 16 tokens):
        // the page offset is wave-uniform and rides in the scalar offset
        const uint32_t pg = __builtin_amdgcn_readfirstlane(pgoff[tp0 + (first >> lgP)]);
        const uint32_t rowbase = pg + static_cast<uint32_t>((first & pmask) * (D / 4));
        td.vh[sub] = ld64(lane_vrow, rowbase + L.off_vhi);
        if (kDense) td.vl[sub] = ld64(lane_vrow, rowbase + L.off_vlo);
        td.vm[sub] = ld32(lane_vmeta, pg + L.off_vmeta + static_cast<uint32_t>((first & pmask) * kNJ * 4));
      } else {
        // 32-token steps may span two 16-token pages: per-lane page offset
        const int tok = first + vslot;
        const uint32_t pg = pgoff[tp0 + (tok >> lgP)];
        const uint32_t ro = pg + static_cast<uint32_t>((tok & pmask) * (D / 4) + 8 * vj);
        td.vh[sub] = ld64(ro, L.off_vhi);
        if (kDense) td.vl[sub] = ld64(ro, L.off_vlo);
        td.vm[sub] = ld32(pg + static_cast<uint32_t>(((tok & pmask) * kNJ + vj) * 4), L.off_vmeta);
      }
    }
    {
      const uint32_t mo = pgoff[tp0 + lane_mpage] + lane_kmeta;
      if (D == 128) {
        const uint2 s2 = ld64(mo, 0), z2 = ld64(mo, 2 * D);
        td.ks[0] = s2.x; td.ks[D / 64 - 1] = s2.y;
        td.kz[0] = z2.x; td.kz[D / 64 - 1] = z2.y;
      } else {
        td.ks[0] = ld32(mo, 0);
        td.kz[0] = ld32(mo, 2 * D);
      }
    }
  };

  // Online softmax against a reference ref = m - kexp * ln 2, where m is the
  // running score maximum and kexp a wave-uniform exponent: every weight is
  // p' = exp(s_t - ref) = p_t * 2^kexp with p_t <= 1, and the value products
  // p' * scale stay in fp16's normal range (below 2^15) for the largest
  // value scale seen so far (kexp falls when a larger scale arrives, like a
  // rising maximum).  lsum, zs and acc carry the same 2^kexp, so the partial
  // (ref, lsum, o) is an ordinary log-sum-exp record.
  float m = -INFINITY, ref = -INFINITY, lsum = 0.0f, zs = 0.0f;
  int kexp = kValComb ? 0 : kMaxWeightExp;
  float acc[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) acc[c] = 0.0f;
  // Candidates collect in LDS (cbuf, n_buf entries).  When a tile's new ones
  // do not fit, the buffer is first re-tested against the running threshold,
  // which only rises; if still full it spills to the global list (n_glob).
  int2* cand_list = a.cand + pair * a.cand_stride + start;
  int n_buf = 0, n_glob = 0;
  auto compact = [&](float th) {
    int n = 0;
    for (int base = 0; base < n_buf; base += 64) {
      const int idx = base + lane;
      int2 e = make_int2(0, 0);
      bool keep = false;
      if (idx < n_buf) {
        e = cbuf[idx];
        keep = __int_as_float(e.y) >= th;
      }
      const uint64_t kb = __ballot(keep);
      // in place: a kept entry moves to n + rank <= idx, never onto an entry
      // not yet read
      if (keep) cbuf[n + __popcll(kb & ((1ull << lane) - 1ull))] = e;
      n += __popcll(kb);
    }
    n_buf = n;
  };
  auto spill = [&]() {
    for (int idx = lane; idx < n_buf; idx += 64) cand_list[n_glob + idx] = cbuf[idx];
    n_glob += n_buf;
    n_buf = 0;
  };

  auto compute = [&](const Tile& cur, int t0) {
    // value metadata of the tile's tokens; rows past the end hold arbitrary
    // bytes, so the last tile of a split zeroes their (scale, zero)
    uint32_t vmeta[kSubs];
#pragma unroll
    for (int sub = 0; sub < kSubs; ++sub) vmeta[sub] = cur.vm[sub];
    if (t0 + kTile > end) {
#pragma unroll
      for (int sub = 0; sub < kSubs; ++sub)
        if (t0 + sub * kSlots + vslot >= end) vmeta[sub] = 0u;
    }
    // --- key metadata of the tile's two key groups -> per-channel multipliers
    float bias0, bias1;
    {
      const bool gvalid = t0 + kGroup * gsel < end;
      float bpart = 0.0f;
#pragma unroll
      for (int c = 0; c < kCPL; ++c) {
        const int d = d0 + c;
        const uint32_t sw = cur.ks[c / 2], zw = cur.kz[c / 2];
        const float s = f16_to_f32((c & 1) ? (sw >> 16) : (sw & 0xffffu));
        const float z = f16_to_f32((c & 1) ? (zw >> 16) : (zw & 0xffffu));
        const float qv = qs[d];
        bpart = fmaf(qv, z, bpart);
        const int pos = (d & ~15) + channel_pos(d & 15);
        qk[gsel][pos] = gvalid ? qv * s * key_factor<kKeyComb>(pos & 15) : 0.0f;
      }
      const float rs = row_sum(gvalid ? bpart : 0.0f);
      bias0 = lane_f(rs, 0) + lane_f(rs, 16);
      bias1 = lane_f(rs, 32) + lane_f(rs, 48);
    }
    __syncthreads();

    // --- scores: one token per lane, keys at the source's full precision
    const int t = t0 + lane;
    const bool valid = t < end;
    float s_t;
    {
      const int g = lane >> 5;
      const float4* qv4 = reinterpret_cast<const float4*>(qk[g]);
      // two interleaved sums: consecutive mixed-precision FMAs never depend
      // on each other, so none waits for its predecessor's result
      float dot0 = 0.0f, dot1 = 0.0f;
      // The next word's multipliers are requested while this word computes
      // where the 16 registers that takes still leave three waves per SIMD
      // (not in the tau = 0 variants, nor for 4-bit sources in the streamed
      // layout); elsewhere each word's are read next to their use.
      constexpr bool kAhead = !kDense && !(kKeyComb && kStreamed);
      float4 mq[4], mq_next[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) mq[v] = qv4[v];
#pragma unroll
      for (int k = 0; k < kWords; ++k) {
        if (kAhead && k + 1 < kWords) {
#pragma unroll
          for (int v = 0; v < 4; ++v) mq_next[v] = qv4[4 * (k + 1) + v];
        }
        const uint32_t hw = (&cur.kh[k / 4].x)[k % 4];
        uint32_t pr[8];
        if (kKeyComb) {
          const uint32_t lw = (&cur.kl[k / 4].x)[k % 4];
          key_pairs_combined(hw, lw, pr);
        } else {
          key_pairs_plain(hw, pr);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          // positions 4v + b of this word: bytes 0, 1, 2, 3 of field v
          const float4 q4 = mq[v];
          dot0 = fmaf(half_lo(pr[2 * v]), q4.x, dot0);
          dot1 = fmaf(half_lo(pr[2 * v + 1]), q4.y, dot1);
          dot0 = fmaf(half_hi(pr[2 * v]), q4.z, dot0);
          dot1 = fmaf(half_hi(pr[2 * v + 1]), q4.w, dot1);
        }
        // each word's work stays together (register pressure): no later
        // word's multiplier reads or unpacking move into it, beyond the
        // next word's reads requested above
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if (k + 1 < kWords) {
#pragma unroll
          for (int v = 0; v < 4; ++v) mq[v] = kAhead ? mq_next[v] : qv4[4 * (k + 1) + v];
        }
      }
      // computed for every lane (no branch): keeps the unrolled reads and
      // arithmetic interleaved instead of sunk into a conditional block
      float dot = dot0 + dot1;
      asm volatile("" : "+v"(dot));
      s_t = valid ? dot + (g ? bias1 : bias0) : -INFINITY;
    }

    // --- online softmax with a wave-uniform running maximum and weight
    //     exponent (fp16 value weights only; tau = 0 weights stay fp32)
    int k_new = kexp;
    if constexpr (!kValComb) {
      // largest value scale of the tile's tokens: fp16 bits of a scale are
      // non-negative, so they order as integers
      uint32_t sb = 0u;
#pragma unroll
      for (int sub = 0; sub < kSubs; ++sub) sb = max(sb, vmeta[sub] & 0xffffu);
      const float smax = f16_to_f32(dpp_wave_max_u32(sb));
      // 2^(14 - floor(log2 smax)) * smax lies in [2^14, 2^15)
      if (smax > 0.0f) k_new = min(k_new, 15 - __builtin_amdgcn_frexp_expf(smax));
    }
    const float tmax = dpp_wave_max_ordered(s_t);
    const float m_new = fmaxf(m, tmax);
    const float ref_new = m_new - static_cast<float>(k_new) * kLn2;
    if (ref_new > ref) {
      const float alpha = __expf(ref - ref_new);
      lsum *= alpha;
      zs *= alpha;
#pragma unroll
      for (int c = 0; c < 32; ++c) acc[c] *= alpha;
      ref = ref_new;
    }
    m = m_new;
    kexp = k_new;
    const float p = valid ? __expf(s_t - ref) : 0.0f;
    lsum += p;
    if (kSparse) {
      // candidates: tokens that pass tau against the LSE of the tokens seen
      // so far (this tile included).  That LSE never exceeds the global one,
      // so no true flag is dropped; the merge kernel takes the exact
      // decision.  The margin covers rounding of this running test.
      const float ltot = dpp_wave_sum(lsum);
      const float theta = ref + logf(ltot) + a.log_tau - 1e-3f;
      const bool f = valid && s_t >= theta;
      const uint64_t bal = __ballot(f);
      const int nb = __popcll(bal);
      if (n_buf + nb > kCandCap) {
        compact(theta);
        if (n_buf + nb > kCandCap) spill();
      }
      if (f) cbuf[n_buf + __popcll(bal & ((1ull << lane) - 1ull))] = make_int2(t, __float_as_int(s_t));
      n_buf += nb;
    }
    ptile[lane] = p;
    __syncthreads();

    // --- values: lane = (token slot, 32-channel group); high plane only
    //     (both planes when tau = 0)
    if constexpr (kValComb) {
#pragma unroll
      for (int sub = 0; sub < kSubs; ++sub) {
        const float pp = ptile[sub * kSlots + vslot];   // 0 for tokens past the end
        const uint32_t meta = vmeta[sub];
        const float vs = f16_to_f32(meta & 0xffffu), vz = f16_to_f32(meta >> 16);
        const float w = pp * vs;
        zs = fmaf(pp, vz, zs);
        const uint32_t hv[2] = {cur.vh[sub].x, cur.vh[sub].y};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          float f[16];
          const uint32_t lv = e ? cur.vl[sub].y : cur.vl[sub].x;
          unpack_combined(hv[e], lv, f);
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[16 * e + q] = fmaf(w, f[q], acc[16 * e + q]);
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // Two value steps at a time: byte k of the two tokens' rows goes into
      // the low bytes of a packed fp16 pair, and a 2-bit field masked in
      // place is an fp16 subnormal code * 4^i * 2^-24 (exact).  One packed
      // dot product then adds w_a * code_a + w_b * code_b in fp32; the
      // weights w = p' * s are rounded to fp16, where the weight exponent
      // keeps them below 2^15 and, for every token whose p_t * s is within
      // 2^-28 of the largest scale seen, above fp16's smallest normal 2^-14
      // (relative rounding error <= 2^-11).  2^24 * 4^-i is applied in the
      // epilogue.
#pragma unroll
      for (int sub = 0; sub < kSubs; sub += 2) {
        float w2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float pp = ptile[(sub + u) * kSlots + vslot];   // 0 for tokens past the end
          const uint32_t meta = vmeta[sub + u];
          const float vs = f16_to_f32(meta & 0xffffu), vz = f16_to_f32(meta >> 16);
          w2[u] = pp * vs;
          zs = kQ4 ? fmaf(pp, fmaf(1.5f, vs, vz), zs)    // bucket centre + zero
                   : fmaf(pp, vz, zs);
        }
        const half2_t wp = {static_cast<_Float16>(w2[0]), static_cast<_Float16>(w2[1])};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t ra = e ? cur.vh[sub].y : cur.vh[sub].x;
          const uint32_t rb = e ? cur.vh[sub + 1].y : cur.vh[sub + 1].x;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            // bytes: [ra.k, 0, rb.k, 0]
            const uint32_t pr = __builtin_amdgcn_perm(rb, ra, 0x0C000C00u | ((4u + k) << 16) | k);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t m = pr & (0x00030003u << (2 * i));
              acc[16 * e + 4 * i + k] =
                  __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, m), wp, acc[16 * e + 4 * i + k], false);
            }
          }
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
  };

  // When all splits run in one round of resident waves, issue priority
  // falls as a split progresses (3, 2, 1 in its first three quarters).
  // Waves sharing a SIMD otherwise issue oldest-first, and with equal splits
  // the youngest finish up to 1.6x later than the oldest; handing priority
  // to the waves that are behind shortens that tail (measured: 3-4% per
  // launch).  In its last quarter a wave's priority is its dispatch rank on
  // its SIMD, so that among waves near their end the youngest, which is
  // behind, issues first instead of the oldest (1-1.5% per step more).  The
  // dispatcher places one wave per SIMD in block order, so the rank is the
  // linear block index over the SIMD count.  Launches of several rounds
  // refill freed slots instead.
  auto set_priority = [](int p) {
    switch (p) {
      case 0: __builtin_amdgcn_s_setprio(0); break;
      case 1: __builtin_amdgcn_s_setprio(1); break;
      case 2: __builtin_amdgcn_s_setprio(2); break;
      default: __builtin_amdgcn_s_setprio(3); break;
    }
  };
  const int n_tiles = (end - start + kTile - 1) / kTile;
  int tiles_done = 0;
  const int lin_block = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int rank = a.grade_simds ? min(3, lin_block / a.grade_simds) : 0;
  auto progress = [&]() {
    ++tiles_done;
    if (a.grade_simds) {
      const int q = (4 * tiles_done) / n_tiles;
      set_priority(q >= 3 ? rank : 3 - q);
    }
  };
  if (a.grade_simds) set_priority(3);

  // ping-pong over two tile buffers: the next tile's loads are issued before
  // the current tile computes.  A tile with no successor issues the same
  // loads over an empty region (no memory traffic) so that every iteration
  // has the same load pattern.
  Tile bufA, bufB;
  fetch(bufA, start, true);
  for (int t0 = start;;) {
    fetch(bufB, t0 + kTile < end ? t0 + kTile : t0, t0 + kTile < end);
    compute(bufA, t0);
    progress();
    t0 += kTile;
    if (t0 >= end) break;
    fetch(bufA, t0 + kTile < end ? t0 + kTile : t0, t0 + kTile < end);
    compute(bufB, t0);
    progress();
    t0 += kTile;
    if (t0 >= end) break;
  }

  // --- partial: sum the token slots of each channel group
#pragma unroll
  for (int c = 0; c < 32; ++c) acc[c] = strided_sum<kNJ>(acc[c]);
  zs = strided_sum<kNJ>(zs);
  lsum = dpp_wave_sum(lsum);
  if (!kSparse && a.direct_out) {
    // The only split of its pair (no tau test to follow): the merge of one
    // record is o / sum, written here, and no merge kernel runs.
    const float inv = 1.0f / lsum;
    if (lane < kNJ) {
#pragma unroll
      for (int c = 0; c < 32; ++c)
        a.out[pair * D + kGroup * lane + 16 * (c / 16) + pos_channel(c % 16)] =
            fmaf(acc[c], kValComb ? inv_unit : dot2_factor(c % 16) * (kQ4 ? 4.0f : 1.0f), zs) * inv;
    }
    if (kDense && a.counters && lane == 0) {   // every low-plane row was read
      const unsigned long long n = static_cast<unsigned long long>(end - start);
      atomicAdd(&a.counters[0], n);
      atomicAdd(&a.counters[1], n * static_cast<unsigned long long>(L.row));
    }
    return;
  }
  if (lane < kNJ) {
#pragma unroll
    for (int c = 0; c < 32; ++c)
      // constant factors kept out of the token loop: the fp8 unit (tau = 0),
      // or the subnormal scale 2^24 * 4^-i; the high plane's weight 4
      part[kPartialPad + kGroup * lane + 16 * (c / 16) + pos_channel(c % 16)] =
          fmaf(acc[c], kValComb ? inv_unit : dot2_factor(c % 16) * (kQ4 ? 4.0f : 1.0f), zs);
  }
  if (lane == 0) {
    part[0] = ref;
    part[1] = lsum;
  }
  if (kSparse) {
    // final test against this split's own LSE (still <= the global one)
    compact(ref + logf(lsum) + a.log_tau - 1e-3f);
    spill();
    if (lane == 0) a.cand_count[pair * a.S + rec] = n_glob;
  }
}

template <int D, int KIND, int MODE>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int T = a.seq_lens[b];
  const int start = split * a.split_len;
  split_segment<D, KIND, MODE, false>(a, b, h, T, start, min(start + a.split_len, T), split, split == 0);
}

// Streamed layout: wave w takes its range of the pairs' tiles laid end to
// end (sequence-major, then head), one split segment per pair it meets.
// The tile counts of all sequences (B <= 256) are scanned once into LDS.
template <int D, int KIND, int MODE>
__global__ __launch_bounds__(64) void decode_stream_kernel(DecodeArgs a) {
  __shared__ int seq_first[kMaxStreamedBatch + 1];   // first tile of each sequence, then the total
  const int lane = threadIdx.x;
  const int H = a.H;
  int own[4], sum = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int bb = 4 * lane + k;
    own[k] = bb < a.batch ? H * ((streamed_len(a, bb) + kTile - 1) / kTile) : 0;
    sum += own[k];
  }
  const int incl = wave_incl_scan(sum);
  int run = incl - sum;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    seq_first[4 * lane + k] = run;
    run += own[k];
  }
  if (lane == 63) seq_first[kMaxStreamedBatch] = run;
  __syncthreads();
  // Wave w takes range w; the last wave then the ranges past the grid.  Only
  // t is carried across segments; the rest is read again from LDS and the
  // arguments (fewer scalars live across the segment's body).
  int t = range_start(a, blockIdx.x);
  while (true) {
    const int total = seq_first[kMaxStreamedBatch];
    const int w = blockIdx.x;
    const int t_end = w == a.waves - 1 ? total : min(range_start(a, w + 1), total);
    if (t >= t_end) break;
    // the sequence holding tile t: the last b < B whose first tile is <= t
    int lo = 0, hi = a.batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seq_first[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    const int b = __builtin_amdgcn_readfirstlane(lo);
    const int first = __builtin_amdgcn_readfirstlane(seq_first[b]);
    const int T = __builtin_amdgcn_readfirstlane(streamed_len(a, b));
    const int nb = (T + kTile - 1) / kTile;                // tiles per head
    const int h = (t - first) / nb;
    const int j = t - first - h * nb;                      // tile index within the pair
    const int wv = wave_of(a, t);                          // w, or a range past the grid
    const int seg = min(nb - j, min(range_start(a, wv + 1), t_end) - t);
    const int rec = wv - wave_of(a, first + h * nb);       // record number within the pair
    split_segment<D, KIND, MODE, true>(a, b, h, T, j * kTile, min((j + seg) * kTile, T), rec, j == 0);
    __syncthreads();                                       // LDS of this segment is free again
    t += seg;
  }
}

template <int D, int KIND, int MODE>
hipError_t launch_typed(const DecodeArgs& a, int batch, hipStream_t stream) {
  const ProfEvents es = prof_events(kClassSplit);
  if (a.streamed)
    hipExtLaunchKernelGGL((decode_stream_kernel<D, KIND, MODE>), dim3(a.waves), dim3(64), 0, stream, es.start,
                          es.stop, 0, a);
  else
    hipExtLaunchKernelGGL((decode_split_kernel<D, KIND, MODE>), dim3(a.S, a.H, batch), dim3(64), 0, stream,
                          es.start, es.stop, 0, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (a.direct_out && MODE != kModeSparse)) return e;
  const ProfEvents em = prof_events(kClassMerge);
  hipExtLaunchKernelGGL((decode_merge_kernel<D, KIND, MODE>), dim3(a.H, batch), dim3(64), 0, stream,
                        em.start, em.stop, 0, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, int batch, int mode, hipStream_t stream) {
  if (a.lay.kind == kKindQ2) return launch_typed<D, kKindQ2, kModePlain>(a, batch, stream);
  if (mode == kModeSparse) return launch_typed<D, kKindQ4, kModeSparse>(a, batch, stream);
  if (mode == kModeDense) return launch_typed<D, kKindQ4, kModeDense>(a, batch, stream);
  return launch_typed<D, kKindQ4, kModePlain>(a, batch, stream);
}

}  // namespace

hipError_t launch_merge_plain(const DecodeArgs& a, int batch, hipStream_t stream) {
  const ProfEvents em = prof_events(kClassMerge);
  if (a.lay.D == 128)
    hipExtLaunchKernelGGL((decode_merge_kernel<128, kKindQ2, kModePlain>), dim3(a.H, batch), dim3(64), 0, stream,
                          em.start, em.stop, 0, a);
  else
    hipExtLaunchKernelGGL((decode_merge_kernel<64, kKindQ2, kModePlain>), dim3(a.H, batch), dim3(64), 0, stream,
                          em.start, em.stop, 0, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int batch, int mode, hipStream_t stream) {
  return a.lay.D == 128 ? launch_d<128>(a, batch, mode, stream) : launch_d<64>(a, batch, mode, stream);
}

}  // namespace lkv
