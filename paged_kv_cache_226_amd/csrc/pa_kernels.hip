// Paged decode attention kernels for gfx950 (CDNA4, wave64, MFMA).
//
// Method (asynchronous-KV-prefetch review, sections 3.2-3.4 and 4.1): a
// work-group owns the block range [s, e) of one (sequence, KV head); its W
// wavefronts walk the range with stride W (wave i takes s+i, s+i+W, ...; the
// KV-cache-prefetching article, section 2.2, gives the same assignment for a
// 4-warp block).  Before computing block j a wavefront issues the fetch of
// block j+W, so the memory latency of the next block overlaps the compute of
// the current one.  Q*K^T is computed per block against Q held in registers,
// then logits times V.
//
// One wavefront serves every query head of its KV head (GQA group g <= 16):
// the heads are the 16 columns of the MFMA tiles, so the per-block cost does
// not grow with g.  Lane l = 16*G + c (lane group G = 0..3, column c = 0..15)
// holds head c.
//
// K block (layout [16 dim groups][16 tokens][8 dims], 4 KiB):
//   Q.K^T = 4 x v_mfma_f32_16x16x32_f16, A = K (16 token rows), B = Q^T.
//   For chunk ch, lane (G, c) loads the 16 bytes of dims 32ch+8G.. of token
//   pi(c) = 4(c%4) + c/4: 1 KiB contiguous per load instruction.  The token
//   permutation pi puts token 4q+G in output row 4G+q, i.e. lane (G, c) ends
//   with the scores of tokens {4q + G : q = 0..3} for head c.
// V block (layout [16 tokens][128 dims], 4 KiB):
//   lane (G, c) loads tokens 4i+G (i = 0..3), dims 8c..8c+7: 1 KiB contiguous
//   per load, and exactly the tokens whose probabilities it holds.
//   O^T += V^T P^T as 8 dim tiles x v_mfma_f32_16x16x16f16; tile t takes dims
//   {8c + t}.  P is split into fp16 hi + lo parts (two MFMAs per tile), so the
//   weights enter with ~22 significant bits; products accumulate in fp32.
//   Lane (G, c) ends with head c, dims 32G..32G+31.
// Softmax: fp32 online softmax per head; the block maximum is shared by the
// four lanes of a column (two cross-lane steps); the accumulator is rescaled
// only when some head's running maximum changed (rescaling by 1 is exact, so
// skipping it changes no bits).
//
// Look-ahead instances (PF): 0 none; 1 an L2 / Infinity-Cache touch of every
// 128 B line of block j+kW (one dword per lane, value discarded); 2 block j+W
// loaded into a second register buffer before block j is computed; 3 both,
// with the touch moved to block j+(1+k)W; 4 the register ring two blocks
// ahead (j+2W); 5 and 6 an LDS ring one and two blocks ahead, filled by
// direct global-to-LDS copies.  k (a.pf_dist, 1..63) is the touch distance
// in iterations; the pages' Algorithm 1 is k = 1.  The arithmetic is the
// same code in every instance, so results are bitwise identical.
//
// Where the slices are: the (block p, KV head h) slice of K starts at byte
// p * k_blk + h * k_head of the K pool (V likewise), so K and V may share a
// pool or be padded; each slice itself has the layout below.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "pa_internal.h"

namespace pa {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;
constexpr int kT = 16;
constexpr int kWave = 64;
constexpr int kBlockHeadBytes = kD * kT * 2;  // 4096
constexpr int kRec = kD + 2;                  // merge record: m, l, o[128]

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Cross-lane steps of the reductions over a column's four lane groups
// (rows of 16 lanes).  v_permlane16_swap exchanges rows 1 and 3 of its first
// operand with rows 0 and 2 of its second, v_permlane32_swap the upper half
// of the first with the lower half of the second.  With x in both operands,
// the pair then holds x of lane l and of lane l ^ 16 (l ^ 32), and f of the
// pair is f(x, x ^ 16) on every lane.  Both are VALU instructions (no LDS
// crossbar); f is commutative here, so the order within the pair does not
// matter and the result is bitwise that of f(x, __shfl_xor(x, 16)).
template <typename F>
__device__ __forceinline__ float xor16_combine(float x, F f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return f(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
template <typename F>
__device__ __forceinline__ float xor32_combine(float x, F f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return f(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float fmax2(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ float fadd2(float a, float b) { return a + b; }
// max / sum over the 4 lanes l, l ^ 16, l ^ 32, l ^ 48
__device__ __forceinline__ float column_max(float x) {
  return xor32_combine(xor16_combine(x, fmax2), fmax2);
}
__device__ __forceinline__ float column_sum(float x) {
  return xor32_combine(xor16_combine(x, fadd2), fadd2);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// Two fp16 values, one from each source dword: half h (0 = low, 1 = high) of
// `lo` into the low half of the result, half h of `hi` into the high half.
__device__ __forceinline__ uint32_t pick_halves(uint32_t lo, uint32_t hi, int h) {
  return __builtin_amdgcn_perm(hi, lo, h ? 0x07060302u : 0x05040100u);
}

// One block as loaded by a lane.  fp16 cache: k[ch] = token pi(c), dims
// 32ch+8G..+7 and v[i] = token 4i+G, dims 8c..8c+7.  FP8 (E4M3) cache:
// k[m] = token pi(c), dims 64m+16G..+15 and v[i] = token 4i+G, dims
// 8c..8c+7, one byte each.
template <bool KV8>
struct BlockBuf {
  u32x4 k[4];
  u32x4 v[4];
};
template <>
struct BlockBuf<true> {
  u32x4 k[2];
  u32x2 v[4];
};

// Eight E4M3 values (two dwords, lowest byte first) widened to fp16.  Every
// E4M3 value is exactly representable in fp16, and the conversion scale is
// 1, so this step is exact; the cache scales are applied to the scores and
// to the output instead.
__device__ __forceinline__ u32x4 widen_fp8x8(uint32_t w0, uint32_t w1) {
  return u32x4{
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true))};
}

// Bytes 0-1 (HIGH false) or 2-3 (HIGH true) of an E4M3 dword widened to an
// fp16 pair, lowest byte in the low half (exact, like widen_fp8x8).
template <bool HIGH>
__device__ __forceinline__ uint32_t widen_fp8x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HIGH));
}

// Pointers of the direct global-to-LDS copy; its cache policy is
// non-temporal, like the direct loads.
typedef __attribute__((address_space(1))) const void gbyte;
typedef __attribute__((address_space(3))) void lbyte;
constexpr int kCachePolicyNT = 2;

// Compile-time flags for the block compute: may the block be a sequence's
// partial last block?
template <bool V>
struct Flag {
  static constexpr bool value = V;
};
constexpr Flag<false> kNoTail{};
constexpr Flag<true> kMayTail{};

// First of the 8 dims that MFMA chunk ch of Q.K^T covers in lane group lg.
// The dot product sums over dims, so K and Q only need the same mapping;
// each cache layout uses the one that its 128-bit loads deliver.
template <bool KV8>
__device__ __forceinline__ int chunk_dim(int ch, int lg) {
  return KV8 ? 64 * (ch >> 1) + 16 * lg + 8 * (ch & 1) : 32 * ch + 8 * lg;
}

// ---------------------------------------------------------------------------
// Walks blocks [s, e) of (sequence b, KV head kvh) with the W waves of the
// work-group (wave w takes s+w, s+w+W, ...) and leaves one record
// (m, l, o[128]) per wave and query head in merge_s.  Every thread of the
// work-group calls it; it synchronises the work-group.
template <int PF, bool DBG, bool KV8>
__device__ __forceinline__ void walk_range(const DecodeArgs& a, const int b, const int kvh,
                                           const int ctx, const int s, const int e,
                                           int32_t* bt_s, float* merge_s) {
  const int G = a.G;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int W = blockDim.x / kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lg = lane >> 4;                    // lane group 0..3
  const int c = lane & 15;                     // column: head c of the group
  const int pic = ((c & 3) << 2) | (c >> 2);   // token held in K row c

  // Stage the range's block-table slice in LDS.
  const int32_t* bt_row = a.bt + (int64_t)b * a.MB;
  for (int i = tid; i < e - s; i += blockDim.x) bt_s[i] = bt_row[s + i];

  // Q^T operand: lane (lg, c), chunk ch = 8 dims of head c starting at
  // chunk_dim(ch, lg) (zero for the padding columns c >= G).
  half8_t qb[4];
  {
    const int hc = c < G ? c : 0;
    const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + kvh * G + hc) * kD;
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      u32x4 w4 = {0u, 0u, 0u, 0u};
      if (c < G) w4 = *reinterpret_cast<const u32x4*>(qrow + chunk_dim<KV8>(ch, lg));
      qb[ch] = __builtin_bit_cast(half8_t, w4);
    }
  }
  __syncthreads();

  float m = -INFINITY;  // running max of head c (log2 units), same in the 4 lanes
  float l = 0.f;        // this lane's share of the softmax denominator
  f32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int kHeadBytes = KV8 ? kBlockHeadBytes / 2 : kBlockHeadBytes;
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(a.k) + kvh * a.k_head;
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(a.v) + kvh * a.v_head;
  const int k_off = (lg * kT + pic) * 16;      // the 16-byte piece of K row pic
  const int v_off = lane * (KV8 ? 8 : 16);     // token lg, dims 8c..8c+7
  typedef BlockBuf<KV8> Buf;

  // K/V are streamed: every byte is used once, by this wave, so the loads
  // are non-temporal (they do not displace lines that will be reused).  The
  // L2 touch of the look-ahead modes is an ordinary load: it is meant to
  // leave its lines in the cache.
  // Every load instruction reads 1 KiB (fp16) or 512 B / 1 KiB (FP8 V / K)
  // of contiguous memory.
  auto load_block = [&](Buf& buf, int64_t ph) {
    const unsigned char* kb = kbase + ph * a.k_blk + k_off;
    const unsigned char* vb = vbase + ph * a.v_blk + v_off;
    if constexpr (KV8) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        buf.k[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + 1024 * i));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        buf.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vb + 512 * i));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        buf.k[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + 1024 * i));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        buf.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + 1024 * i));
    }
  };

  // One dword per lane: lanes 0-31 cover the 128 B lines of the K block
  // (32 fp16 / 16 FP8), lanes 32-63 those of the V block.
  auto touch_block = [&](int64_t ph) -> uint32_t {
    constexpr int kLines = kHeadBytes / 128;
    const unsigned char* base = lane < 32 ? kbase + ph * a.k_blk : vbase + ph * a.v_blk;
    return *reinterpret_cast<const uint32_t*>(base + (lane & (kLines - 1)) * 128);
  };

  auto trace_put = [&](int j, int slot, int value) {
    if (DBG && a.dbg_trace && lane == 0)
      a.dbg_trace[(((int64_t)b * a.Hkv + kvh) * a.MB + j) * 2 + slot] = value;
  };

  // `MayTail` is false wherever the block cannot be the sequence's last one
  // (every steady-state iteration: those always leave blocks for later
  // iterations of the same wave).  Without the masking branch there the
  // loaded registers are used as they are, and the compiler has no reason to
  // copy a look-ahead buffer, a copy that would wait for its loads early.
  auto compute = [&](Buf& buf, int j, auto may_tail) {
    constexpr bool MayTail = decltype(may_tail)::value;
    // fp16 operands: K chunks and V rows (an E4M3 V stays in bytes until the
    // P.V operands are built)
    u32x4 kh[4], vh[4];
    u32x2 vb[4];
    if constexpr (KV8) {
#pragma unroll
      for (int ch = 0; ch < 4; ++ch)
        kh[ch] = widen_fp8x8(buf.k[ch >> 1][2 * (ch & 1)], buf.k[ch >> 1][2 * (ch & 1) + 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i) vb[i] = buf.v[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kh[i] = buf.k[i];
        vh[i] = buf.v[i];
      }
    }
    if (DBG && a.dbg_k) {
      unsigned char* dst = reinterpret_cast<unsigned char*>(a.dbg_k) +
                           ((((int64_t)b * a.Hkv + kvh) * a.MB + j) * kT + pic) * kD * 2;
#pragma unroll
      for (int ch = 0; ch < 4; ++ch)
        *reinterpret_cast<u32x4*>(dst + 2 * chunk_dim<KV8>(ch, lg)) = kh[ch];
    }
    const int rem = ctx - j * kT;  // valid tokens in this block, >= 1
    const bool tail = MayTail && rem < kT;
    if (tail) {  // tokens past the context: V zero (E4M3 0 widens to +0)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * i + lg >= rem) {
          if constexpr (KV8)
            vb[i] = u32x2{0u, 0u};
          else
            vh[i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
    // scores of tokens 4q+lg for head c
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ch = 0; ch < 4; ++ch)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, kh[ch]),
                                                     qb[ch], sacc, 0, 0, 0);
    float sc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) sc[q] = sacc[q] * a.scale_log2;
    if (tail) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (4 * q + lg >= rem) sc[q] = -INFINITY;
    }
    float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    bm = column_max(bm);
    const float m_new = fmaxf(m, bm);  // finite: every block has a valid token
    const float alpha = fast_exp2(m - m_new);
    float pr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) pr[q] = fast_exp2(sc[q] - m_new);
    l = l * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    m = m_new;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] *= alpha;
    }
    half4_t phi, plo;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      phi[q] = (_Float16)pr[q];
      plo[q] = (_Float16)(pr[q] - (float)phi[q]);
    }
    // Tile t takes dim t (of this lane's 8) of tokens 0..3 of the lane group:
    // (token 0, token 1) in the low dword, (token 2, token 3) in the high.
    auto pv_tile = [&](int t, uint32_t lo, uint32_t hi) {
      const half4_t av = __builtin_bit_cast(half4_t, u32x2{lo, hi});
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, phi, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, plo, acc[t], 0, 0, 0);
    };
    if constexpr (KV8) {
      // One byte permute puts dims t and t+1 of two tokens in token order
      // (t0.d, t1.d, t0.d+1, t1.d+1), so each conversion yields a tile's
      // pair directly: 8 permutes and 16 conversions per block instead of
      // widening every row (16) and then permuting the halves (16).
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        const int b0 = t & 3;
        const uint32_t sel = b0 | (4 + b0) << 8 | (b0 + 1) << 16 | (5 + b0) << 24;
        const uint32_t w01 = __builtin_amdgcn_perm(t < 4 ? vb[1].x : vb[1].y,
                                                   t < 4 ? vb[0].x : vb[0].y, sel);
        const uint32_t w23 = __builtin_amdgcn_perm(t < 4 ? vb[3].x : vb[3].y,
                                                   t < 4 ? vb[2].x : vb[2].y, sel);
        pv_tile(t, widen_fp8x2<false>(w01), widen_fp8x2<false>(w23));
        pv_tile(t + 1, widen_fp8x2<true>(w01), widen_fp8x2<true>(w23));
      }
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int u = t >> 1, h = t & 1;
        pv_tile(t, pick_halves(vh[0][u], vh[1][u], h), pick_halves(vh[2][u], vh[3][u], h));
      }
    }
  };

  // ---- the block walk -----------------------------------------------------
  // Wave `wave` runs n_it iterations; iteration it computes block j0 + it*W,
  // whose table entry is bt_s[wave + it*W].  The entries of iterations
  // [base, base+64) and [base+64, base+128) are held one per lane in btv0 /
  // btv1 and read with v_readlane, so no block address waits on memory; the
  // pair moves on by 64 when the walk crosses a chunk.
  const int j0 = s + wave;
  const int n_it = j0 < e ? (e - j0 + W - 1) / W : 0;
  const int nslice = e - s;
  auto bt_chunk = [&](int base) -> int {
    const int idx = wave + W * (base + lane);
    return idx < nslice ? bt_s[idx] : 0;
  };
  int chunk_base = 0;
  int btv0 = bt_chunk(0);
  int btv1 = bt_chunk(64);
  auto phys_it = [&](int it) -> int64_t {
    const int v0 = __builtin_amdgcn_readlane(btv0, it & 63);
    const int v1 = __builtin_amdgcn_readlane(btv1, it & 63);
    int ph = it - chunk_base < 64 ? v0 : v1;
    if (DBG) {
      if (ph < 0 || (int64_t)ph >= a.NB) {
        if (lane == 0 && a.dbg_err) atomicOr(a.dbg_err, 1);
        ph = 0;
      }
    }
    return (int64_t)ph;
  };
  auto advance = [&](int it) {
    if (((it + 1) & 63) == 0) {
      chunk_base += 64;
      btv0 = btv1;
      btv1 = bt_chunk(chunk_base + 64);
    }
  };
  uint32_t sink = 0;

  // The steady-state loops issue their look-ahead loads unconditionally (the
  // last iterations are peeled), so the compiler's wait before block j's
  // first use counts block j+W's loads as still in flight.
  if constexpr (PF <= 1) {
    uint32_t pend = 0;
    int it = 0;
    for (; it + 1 < n_it; ++it) {  // block j+W exists
      const int j = j0 + it * W;
      Buf buf;
      // All of block j's loads (and the touch) are issued before its compute
      // starts; unfenced, the compiler issues the V loads only after the
      // first K load has arrived, which serialises two latencies.
      __builtin_amdgcn_sched_barrier(0);
      load_block(buf, phys_it(it));
      uint32_t got = 0;
      if (PF == 1 && it + a.pf_dist < n_it) {
        got = touch_block(phys_it(it + a.pf_dist));
        trace_put(j + a.pf_dist * W, 1, wave);
      }
      __builtin_amdgcn_sched_barrier(0);
      trace_put(j, 0, (wave << 16) | it);
      compute(buf, j, kNoTail);
      if (PF == 1) {
        sink ^= pend;
        pend = got;
      }
      advance(it);
    }
    if (it < n_it) {  // this wave's last block: nothing left to fetch ahead
      const int j = j0 + it * W;
      Buf buf;
      load_block(buf, phys_it(it));
      trace_put(j, 0, (wave << 16) | it);
      compute(buf, j, kMayTail);
    }
    sink ^= pend;
  } else if constexpr (PF == 5 || PF == 6) {
    // LDS ring of depth D: block j+D*W is copied by the direct global-to-LDS
    // path (global_load_lds_dwordx4, no registers involved) into one of this
    // wave's D+1 LDS slots while block j is read out of another and
    // computed.  The copy keeps the slice's byte order (1 KiB contiguous per
    // instruction); the read-back takes the same per-lane pieces as the
    // direct loads.  Holding the look-ahead blocks in LDS instead of
    // registers frees about 32 VGPRs per lane and block.
    constexpr int D = PF - 4;
    constexpr int kSlot = 2 * kHeadBytes;             // one block's K and V
    constexpr int kCopies = 2 * (kHeadBytes / 1024);  // copy instructions per block
    unsigned char* const ring = reinterpret_cast<unsigned char*>(merge_s) + wave * (D + 1) * kSlot;
    auto dma_block = [&](int64_t ph, unsigned char* slot) {
      const unsigned char* ks = kbase + ph * a.k_blk + lane * 16;
      const unsigned char* vs = vbase + ph * a.v_blk + lane * 16;
#pragma unroll
      for (int q = 0; q < kHeadBytes / 1024; ++q) {
        __builtin_amdgcn_global_load_lds((gbyte*)(ks + 1024 * q),
                                         (lbyte*)(slot + 1024 * q), 16, 0,
                                         kCachePolicyNT);
        __builtin_amdgcn_global_load_lds((gbyte*)(vs + 1024 * q),
                                         (lbyte*)(slot + kHeadBytes + 1024 * q),
                                         16, 0, kCachePolicyNT);
      }
    };
    auto read_block = [&](Buf& buf, const unsigned char* slot) {
      const unsigned char* kb = slot + k_off;
      const unsigned char* vb = slot + kHeadBytes + v_off;
      if constexpr (KV8) {
#pragma unroll
        for (int i = 0; i < 2; ++i) buf.k[i] = *reinterpret_cast<const u32x4*>(kb + 1024 * i);
#pragma unroll
        for (int i = 0; i < 4; ++i) buf.v[i] = *reinterpret_cast<const u32x2*>(vb + 512 * i);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) buf.k[i] = *reinterpret_cast<const u32x4*>(kb + 1024 * i);
#pragma unroll
        for (int i = 0; i < 4; ++i) buf.v[i] = *reinterpret_cast<const u32x4*>(vb + 1024 * i);
      }
    };
    // The waits are explicit: the copies are memory writes whose completion
    // only the vector-memory counter reports, in issue order.  Before a slot
    // is refilled its reads must have returned (lgkmcnt 0); before a slot is
    // read its copy must have landed, which with the D later blocks' copies
    // issued after it is vmcnt <= D * kCopies (other vector memory operations
    // issued in between only make the wait stricter).
    // block it of this wave lives in slot it mod (D+1)
    int slot_cur = 0;  // slot of iteration it
    int slot_new = D;  // slot of the next copy, block it+D
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (d < n_it) dma_block(phys_it(d), ring + d * kSlot);
    int it = 0;
    for (; it + D < n_it; ++it) {
      const int j = j0 + it * W;
      Buf buf;
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      dma_block(phys_it(it + D), ring + slot_new * kSlot);
      if constexpr (D * kCopies == 16)
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      else if constexpr (D * kCopies == 8)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      read_block(buf, ring + slot_cur * kSlot);
      __builtin_amdgcn_sched_barrier(0);
      trace_put(j + D * W, 1, wave);
      trace_put(j, 0, (wave << 16) | it);
      compute(buf, j, kNoTail);
      advance(it);
      slot_cur = slot_cur == D ? 0 : slot_cur + 1;
      slot_new = slot_new == D ? 0 : slot_new + 1;
    }
    // this wave's last D blocks: nothing left to copy ahead; the copies of
    // the blocks after `it` may still be in flight
    for (; it < n_it; ++it) {
      const int j = j0 + it * W;
      Buf buf;
      __builtin_amdgcn_sched_barrier(0);
      if (D == 2 && it + 1 < n_it) {
        if constexpr (kCopies == 8)
          asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else
          asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      read_block(buf, ring + slot_cur * kSlot);
      __builtin_amdgcn_sched_barrier(0);
      trace_put(j, 0, (wave << 16) | it);
      compute(buf, j, kMayTail);
      advance(it);
      slot_cur = slot_cur == D ? 0 : slot_cur + 1;
    }
    // the merge records below overlay the slots of other waves
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
  } else {
    // Register look-ahead of depth D: block j + D*W is fetched into a ring of
    // D+1 buffers while block j is computed.  The steady loop is unrolled
    // D+1 times so every buffer index is a compile-time constant.
    constexpr int D = PF == 4 ? 2 : 1;
    Buf bufs[D + 1];
    uint32_t pend = 0;
    auto step = [&](Buf& cur, Buf& ahead, int it) {  // block it+D exists
      const int j = j0 + it * W;
      // Scheduling fences: the compiler does not model HBM latency.  Without
      // them it starts the next block's Q.K^T right after that block's loads
      // are issued (waiting on the very data the look-ahead is meant to
      // overlap), and issues the look-ahead loads only after the current
      // block has arrived.
      __builtin_amdgcn_sched_barrier(0);
      load_block(ahead, phys_it(it + D));
      __builtin_amdgcn_sched_barrier(0);
      trace_put(j + D * W, 1, wave);
      uint32_t got = 0;
      if (PF == 3 && it + D + a.pf_dist < n_it) got = touch_block(phys_it(it + D + a.pf_dist));
      trace_put(j, 0, (wave << 16) | it);
      compute(cur, j, kNoTail);
      if (PF == 3) {
        sink ^= pend;
        pend = got;
      }
      advance(it);
      __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int u = 0; u < D; ++u)
      if (u < n_it) load_block(bufs[u], phys_it(u));
    int it = 0;
    for (; it + 2 * D < n_it; it += D + 1) {  // iterations it..it+D all fetch ahead
#pragma unroll
      for (int u = 0; u <= D; ++u) step(bufs[u], bufs[(u + D) % (D + 1)], it + u);
    }
    for (; it < n_it; ++it) {  // bufs[0..D-1] hold blocks it..it+D-1
      const int j = j0 + it * W;
      if (it + D < n_it) {
        load_block(bufs[D], phys_it(it + D));
        trace_put(j + D * W, 1, wave);
      }
      uint32_t got = 0;
      if (PF == 3 && it + D + a.pf_dist < n_it) got = touch_block(phys_it(it + D + a.pf_dist));
      trace_put(j, 0, (wave << 16) | it);
      compute(bufs[0], j, kMayTail);
      if (PF == 3) {
        sink ^= pend;
        pend = got;
      }
      advance(it);
#pragma unroll
      for (int u = 0; u < D; ++u) bufs[u] = bufs[u + 1];
    }
    sink ^= pend;
  }
  // The touched data is discarded; this keeps the loads alive without ever
  // storing (a.sink_enable is 0 in every call).
  if (a.sink_enable && sink == 0x9E3779B9u && lane == 0) a.sink[0] = (int32_t)sink;

  // ---- merge: the 4 lanes of a column, then the W waves through LDS -------
  const float lt = column_sum(l);
  if (c < G) {
    float* rec = merge_s + (wave * G + c) * kRec;
    if (lg == 0) {
      rec[0] = m;
      rec[1] = lt;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int t = 0; t < 8; ++t) rec[2 + 32 * lg + 8 * q + t] = acc[t][q];
  }
  __syncthreads();
}


// ---------------------------------------------------------------------------
// The pages' two-loop structure, kept as a comparison for the fused walk
// above (fp16 caches, no debug outputs).  Loop 1 walks the range with a K
// look-ahead and writes the scaled scores of every token to LDS; the
// per-head maximum M of the range is taken between the loops; loop 2 walks
// the range again with a V look-ahead and accumulates exp2(s - M) * V.  Each
// wave leaves the same (m, l, o[128]) record as walk_range, with m = M.
// PF: 0 no look-ahead, 1 L2 touch of the next K (loop 1) / V (loop 2) block,
// 2 register double buffer of the next K / V block, 3 both.
template <int PF>
__device__ __forceinline__ void walk_two_loop(const DecodeArgs& a, const int b, const int kvh,
                                              const int ctx, const int s, const int e,
                                              int32_t* bt_s, float* merge_s, float* logit_s,
                                              float* wmax_s) {
  const int G = a.G;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int W = blockDim.x / kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lg = lane >> 4;
  const int c = lane & 15;
  const int pic = ((c & 3) << 2) | (c >> 2);

  const int32_t* bt_row = a.bt + (int64_t)b * a.MB;
  for (int i = tid; i < e - s; i += blockDim.x) bt_s[i] = bt_row[s + i];
  half8_t qb[4];
  {
    const int hc = c < G ? c : 0;
    const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + kvh * G + hc) * kD;
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      u32x4 w4 = {0u, 0u, 0u, 0u};
      if (c < G) w4 = *reinterpret_cast<const u32x4*>(qrow + chunk_dim<false>(ch, lg));
      qb[ch] = __builtin_bit_cast(half8_t, w4);
    }
  }
  __syncthreads();

  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(a.k) + kvh * a.k_head;
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(a.v) + kvh * a.v_head;
  const int k_off = (lg * kT + pic) * 16;
  const int v_off = lane * 16;
  const int j0 = s + wave;
  const int n_it = j0 < e ? (e - j0 + W - 1) / W : 0;
  // table entry of iteration it (the range's slice is in LDS)
  auto phys_it = [&](int it) -> int64_t { return (int64_t)bt_s[wave + it * W]; };
  auto load4 = [&](u32x4* r, const unsigned char* base, int64_t blk, int64_t ph, int off) {
    const unsigned char* p = base + ph * blk + off;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 1024 * i));
  };
  // one dword of each 128 B line of a 4 KiB K or V block
  auto touch = [&](const unsigned char* base, int64_t blk, int64_t ph) -> uint32_t {
    return *reinterpret_cast<const uint32_t*>(base + ph * blk + (lane & 31) * 128);
  };
  uint32_t sink = 0;

  // ---- loop 1: scores ------------------------------------------------------
  float m = -INFINITY;
  auto scores = [&](const u32x4* kh, int j) {
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ch = 0; ch < 4; ++ch)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, kh[ch]), qb[ch],
                                                     sacc, 0, 0, 0);
    const int rem = ctx - j * kT;
    float bm = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float sc = 4 * q + lg < rem ? sacc[q] * a.scale_log2 : -INFINITY;
      bm = fmaxf(bm, sc);
      if (c < G) logit_s[((j - s) * kT + 4 * q + lg) * G + c] = sc;
    }
    bm = column_max(bm);
    m = fmaxf(m, bm);
  };
  if constexpr (PF >= 2) {
    u32x4 ka[4], kb[4];
    if (n_it > 0) load4(ka, kbase, a.k_blk, phys_it(0), k_off);
    int it = 0;
    for (; it + 2 < n_it; it += 2) {
      __builtin_amdgcn_sched_barrier(0);
      load4(kb, kbase, a.k_blk, phys_it(it + 1), k_off);
      if (PF == 3 && it + 2 < n_it) sink ^= touch(kbase, a.k_blk, phys_it(it + 2));
      __builtin_amdgcn_sched_barrier(0);
      scores(ka, j0 + it * W);
      __builtin_amdgcn_sched_barrier(0);
      load4(ka, kbase, a.k_blk, phys_it(it + 2), k_off);
      if (PF == 3 && it + 3 < n_it) sink ^= touch(kbase, a.k_blk, phys_it(it + 3));
      __builtin_amdgcn_sched_barrier(0);
      scores(kb, j0 + (it + 1) * W);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (; it < n_it; ++it) {
      if (it + 1 < n_it) load4(kb, kbase, a.k_blk, phys_it(it + 1), k_off);
      scores(ka, j0 + it * W);
#pragma unroll
      for (int i = 0; i < 4; ++i) ka[i] = kb[i];
    }
  } else {
    for (int it = 0; it < n_it; ++it) {
      u32x4 kh[4];
      __builtin_amdgcn_sched_barrier(0);
      load4(kh, kbase, a.k_blk, phys_it(it), k_off);
      if (PF == 1 && it + 1 < n_it) sink ^= touch(kbase, a.k_blk, phys_it(it + 1));
      __builtin_amdgcn_sched_barrier(0);
      scores(kh, j0 + it * W);
    }
  }

  // ---- the range maximum of each head -------------------------------------
  if (lg == 0 && c < G) wmax_s[wave * G + c] = m;
  __syncthreads();
  float M = -INFINITY;
  for (int w = 0; w < W; ++w) M = fmaxf(M, wmax_s[w * G + (c < G ? c : 0)]);
  // M is finite: the range holds at least one valid token

  // ---- loop 2: weights times V ---------------------------------------------
  float l = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto weigh = [&](u32x4* vh, int j) {
    const int rem = ctx - j * kT;
    half4_t phi, plo;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float pr = 0.f;
      if (c < G) pr = fast_exp2(logit_s[((j - s) * kT + 4 * q + lg) * G + c] - M);
      l += pr;
      phi[q] = (_Float16)pr;
      plo[q] = (_Float16)(pr - (float)phi[q]);
    }
    if (rem < kT) {  // a partial last block: its unused V slots may hold anything
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * i + lg >= rem) vh[i] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int u = t >> 1, h = t & 1;
      u32x2 vt;
      vt.x = pick_halves(vh[0][u], vh[1][u], h);
      vt.y = pick_halves(vh[2][u], vh[3][u], h);
      const half4_t av = __builtin_bit_cast(half4_t, vt);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, phi, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, plo, acc[t], 0, 0, 0);
    }
  };
  if constexpr (PF >= 2) {
    u32x4 va[4], vb[4];
    if (n_it > 0) load4(va, vbase, a.v_blk, phys_it(0), v_off);
    int it = 0;
    for (; it + 2 < n_it; it += 2) {
      __builtin_amdgcn_sched_barrier(0);
      load4(vb, vbase, a.v_blk, phys_it(it + 1), v_off);
      if (PF == 3 && it + 2 < n_it) sink ^= touch(vbase, a.v_blk, phys_it(it + 2));
      __builtin_amdgcn_sched_barrier(0);
      weigh(va, j0 + it * W);
      __builtin_amdgcn_sched_barrier(0);
      load4(va, vbase, a.v_blk, phys_it(it + 2), v_off);
      if (PF == 3 && it + 3 < n_it) sink ^= touch(vbase, a.v_blk, phys_it(it + 3));
      __builtin_amdgcn_sched_barrier(0);
      weigh(vb, j0 + (it + 1) * W);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (; it < n_it; ++it) {
      if (it + 1 < n_it) load4(vb, vbase, a.v_blk, phys_it(it + 1), v_off);
      weigh(va, j0 + it * W);
#pragma unroll
      for (int i = 0; i < 4; ++i) va[i] = vb[i];
    }
  } else {
    for (int it = 0; it < n_it; ++it) {
      u32x4 vh[4];
      __builtin_amdgcn_sched_barrier(0);
      load4(vh, vbase, a.v_blk, phys_it(it), v_off);
      if (PF == 1 && it + 1 < n_it) sink ^= touch(vbase, a.v_blk, phys_it(it + 1));
      __builtin_amdgcn_sched_barrier(0);
      weigh(vh, j0 + it * W);
    }
  }
  if (a.sink_enable && sink == 0x9E3779B9u && lane == 0) a.sink[0] = (int32_t)sink;

  // ---- records: the same layout as walk_range ------------------------------
  const float lt = column_sum(l);
  if (c < G) {
    float* rec = merge_s + (wave * G + c) * kRec;
    if (lg == 0) {
      rec[0] = M;
      rec[1] = lt;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int t = 0; t < 8; ++t) rec[2 + 32 * lg + 8 * q + t] = acc[t][q];
  }
  __syncthreads();
}

// Softmax-merge of the W wave records of head h: running max M (log2 units),
// denominator L and unnormalised output O for dim d.
__device__ __forceinline__ void combine_waves(const float* merge_s, int W, int G, int h, int d,
                                              float& M, float& L, float& O) {
  M = -INFINITY;
  for (int w = 0; w < W; ++w) M = fmaxf(M, merge_s[(w * G + h) * kRec]);
  const float Mu = M == -INFINITY ? 0.f : M;
  L = 0.f;
  O = 0.f;
  for (int w = 0; w < W; ++w) {
    const float* rec = merge_s + (w * G + h) * kRec;
    const float al = fast_exp2(rec[0] - Mu);
    L += al * rec[1];
    O += al * rec[2 + d];
  }
}

// ---------------------------------------------------------------------------
// Longest-first dispatch.  Work-groups start in grid order, so grid row r
// takes the sequence with the r-th most blocks (ties by index): the longest
// sequences start first and the short ones fill in behind them, which
// shortens the tail of a ragged batch.  Every work-group ranks the B block
// counts itself (B <= 256, so at most 64 16-byte LDS reads per thread); the
// ranks are a permutation of 0..B-1, so exactly one sequence matches r.
// When every sequence has the same block count the ranking is the identity
// (ties go by index) and the scan is skipped: on uniform batches it cost
// up to 4 % (GQA 32/8, batch 128 x 1K tokens: 78.2 % of the HBM peak
// ranked, 81.4 % with the shortcut, 81.9 % in natural order).
__device__ __forceinline__ int ranked_sequence(const DecodeArgs& a, int r, int tab_tokens,
                                            unsigned char* smem) {
  int* nb_s = reinterpret_cast<int*>(smem);
  const int Bp = (a.B + 3) / 4 * 4;
  int* sel_s = nb_s + Bp;
  const int tid = threadIdx.x;
  for (int i = tid; i < Bp; i += blockDim.x) {
    int c = i < a.B ? a.ctx[i] : 0;
    c = c < 0 ? 0 : (c > tab_tokens ? tab_tokens : c);
    nb_s[i] = i < a.B ? (c + kT - 1) / kT : -1;  // padding never outranks
  }
  __syncthreads();
  int differs = 0;
  for (int i = tid; i < a.B; i += blockDim.x) differs |= nb_s[i] != nb_s[0];
  if (!__syncthreads_or(differs)) return r;  // the barrier also ends the LDS reads
  for (int i = tid; i < a.B; i += blockDim.x) {
    const int ki = nb_s[i];
    int rank = 0;
    for (int j = 0; j < Bp; j += 4) {
      const int4 k4 = *reinterpret_cast<const int4*>(nb_s + j);
      rank += (k4.x > ki) | ((k4.x == ki) & (j < i));
      rank += (k4.y > ki) | ((k4.y == ki) & (j + 1 < i));
      rank += (k4.z > ki) | ((k4.z == ki) & (j + 2 < i));
      rank += (k4.w > ki) | ((k4.w == ki) & (j + 3 < i));
    }
    if (rank == r) *sel_s = i;
  }
  __syncthreads();
  const int b = *sel_s;
  __syncthreads();  // the LDS is reused by the block walk
  return b;
}

// ---------------------------------------------------------------------------
// Balanced split.  With ragged contexts and fewer (sequence, KV head) pairs
// than CUs, fixed-size partitions leave the longest sequences' partitions
// running alone on their CUs long after the rest have finished (a CU reads
// at most about 130 x 128 B in flight).  Here every work-group of KV head
// kvh reads all B context lengths and takes the same decision: the
// partition size PB is the smallest multiple of the wave count W in
// [a.PB, a.pb_max] for which all sequences together need at most a.nslot
// partitions and no sequence needs more than a.P (the workspace's partition
// stride) and, unless partitions hold at least kReduceBigPartition blocks,
// none needs more than the reduce merges in one round trip (kReduceRegs);
// grid row y then takes partition y of the list (sequence 0's
// partitions first, then sequence 1's, ...) or nothing.  Each wave computes it
// (B <= 256: lane l of each wave holds sequences 4l..4l+3).
struct Slot {
  int b, p, np, pb;  // sequence, its partition index and count, blocks per partition
  int ctx;           // the sequence's context length as stored
};

// Sum over the 64 lanes, in every lane, without the LDS crossbar: DPP
// rotations and quad permutes within each row of 16 lanes, then the row
// swaps v_permlane16_swap / v_permlane32_swap across rows.
__device__ __forceinline__ int wave_sum_i32(int x) {
  x += __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);  // row_ror:8
  x += __builtin_amdgcn_mov_dpp(x, 0x124, 0xF, 0xF, false);  // row_ror:4
  x += __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  x += __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  const auto r16 = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  x = (int)r16[0] + (int)r16[1];
  const auto r32 = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  return (int)r32[0] + (int)r32[1];
}

// Maximum over the 64 lanes, in every lane (same steps as wave_sum_i32).
__device__ __forceinline__ int wave_max_i32(int x) {
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false));  // row_ror:8
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0x124, 0xF, 0xF, false));  // row_ror:4
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  const auto r16 = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  x = max((int)r16[0], (int)r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  return max((int)r32[0], (int)r32[1]);
}

// Inclusive prefix sum over the 64 lanes: row-local shifts (lanes shifted in
// from outside the row add 0), then the last lane of each row broadcast into
// the rows after it.
__device__ __forceinline__ int wave_prefix_i32(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// ceil(n / d) for 0 <= n < 2^24, 1 <= d < 2^24: a float estimate corrected
// to the exact quotient (cheaper than the integer division sequence).
__device__ __forceinline__ int ceil_div_small(int n, int d, float rd) {
  const int x = n + d - 1;
  int q = (int)((float)x * rd);
  if ((q + 1) * d <= x) ++q;
  if (q * d > x) --q;
  return q;
}

// Every wave computes the same slot (the inputs are the same and the
// arithmetic is deterministic), so no LDS or barrier is needed to share it.
__device__ Slot balanced_slot(const DecodeArgs& a, int slot, int tab_tokens) {
  const int lane = threadIdx.x & (kWave - 1);
  const int W = blockDim.x / kWave;
  int nb[4], raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = 4 * lane + i;
    raw[i] = idx < a.B ? a.ctx[idx] : 0;
    const int c = raw[i] < 0 ? 0 : (raw[i] > tab_tokens ? tab_tokens : raw[i]);
    nb[i] = (c + kT - 1) / kT;
  }
  int pb;
  const int nb0 = __builtin_amdgcn_readfirstlane(nb[0]);
  bool same = true;
#pragma unroll
  for (int i = 0; i < 4; ++i) same &= 4 * lane + i >= a.B || nb[i] == nb0;
  if (__builtin_amdgcn_ballot_w64(!same) == 0) {
    // every sequence has nb0 blocks and may take a.k_uniform = min(nslot / B,
    // P) partitions: the size is the smallest step multiple >= nb0 / that,
    // and >= the reduce bound below
    pb = ceil_div_small(nb0, a.k_uniform, 1.0f / (float)a.k_uniform);
    const int red = (nb0 + kReduceRegs - 1) / kReduceRegs;
    const int red_lo = red < kReduceBigPartition ? red : kReduceBigPartition;
    pb = pb < red_lo ? red_lo : pb;
    pb = (pb + W - 1) / W * W;
    pb = pb < a.PB ? a.PB : (pb > a.pb_max ? a.pb_max : pb);
  } else {
    auto parts = [&](int size) {  // partitions of `size` blocks over all sequences
      const float rd = 1.0f / (float)size;
      int n = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) n += ceil_div_small(nb[i], size, rd);
      return wave_sum_i32(n);
    };
    // The count falls as the size grows, and the host sized nslot so that
    // pb_max always fits.  With T blocks over B' non-empty sequences, a
    // size below T / nslot cannot fit and one of T / (nslot - B') always
    // does (each sequence adds at most one partly filled partition), so
    // the search starts from that bracket.
    int t = 0, ne = 0, mx = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      t += nb[i];
      ne += nb[i] > 0;
      mx = nb[i] > mx ? nb[i] : mx;
    }
    t = wave_sum_i32(t);
    ne = wave_sum_i32(ne);
    mx = wave_max_i32(mx);
    // a size below ceil(mx / P) would give the longest sequence more
    // partitions than the workspace holds; one below min(64, ceil(mx / 8))
    // more than the reduce merges in one round trip, in small partitions
    const int lo_p = (mx + a.P - 1) / a.P;
    const int red = (mx + kReduceRegs - 1) / kReduceRegs;
    const int red_lo = red < kReduceBigPartition ? red : kReduceBigPartition;
    int lo = (t + a.nslot - 1) / a.nslot;
    lo = lo < lo_p ? lo_p : lo;
    lo = lo < red_lo ? red_lo : lo;
    int hi = a.nslot > ne ? (t + (a.nslot - ne) - 1) / (a.nslot - ne) : a.pb_max;
    hi = hi < lo ? lo : hi;
    lo = (lo + W - 1) / W;  // in units of W
    hi = (hi + W - 1) / W;
    lo = lo < a.PB / W ? a.PB / W : lo;
    hi = hi > a.pb_max / W ? a.pb_max / W : hi;
    hi = hi < lo ? lo : hi;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (parts(mid * W) <= a.nslot)
        hi = mid;
      else
        lo = mid + 1;
    }
    pb = lo * W;
  }
  const float rd = 1.0f / (float)pb;
  int np[4], mine = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    np[i] = ceil_div_small(nb[i], pb, rd);
    mine += np[i];
  }
  int start = wave_prefix_i32(mine) - mine;  // partitions of the lanes before
  int found = -1, fp = 0, fnp = 0, fctx = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (slot >= start && slot < start + np[i]) {
      found = 4 * lane + i;
      fp = slot - start;
      fnp = np[i];
      fctx = raw[i];
    }
    start += np[i];
  }
  // at most one lane holds the slot; move its values to every lane
  const uint64_t owner = __builtin_amdgcn_ballot_w64(found >= 0);
  Slot r = {-1, 0, 0, pb, 0};
  if (owner) {
    const int ol = __builtin_ctzll(owner);
    r.b = __builtin_amdgcn_readlane(found, ol);
    r.p = __builtin_amdgcn_readlane(fp, ol);
    r.np = __builtin_amdgcn_readlane(fnp, ol);
    r.ctx = __builtin_amdgcn_readlane(fctx, ol);
  }
  return r;
}

// Even split: this work-group's share [X, Y) of a sequence of positions in
// which every non-empty (KV head, sequence) unit takes K + nb positions, K
// the cost of a piece change in blocks (a.even_kappa) and nb its blocks at
// positions [v + K, v + K + nb) from its start v.  Units are KV-head-major:
// head kvh's fill [kvh N, (kvh + 1) N), N = sum of (K + nb) over the
// non-empty sequences, T = Hkv N.  (Sequence-major order, a sequence's KV
// heads one after the other, measured 5-7 % slower: the work-groups that
// run at the same time then read every other KV head's slice of the same
// blocks instead of all of them.)  Every wave finds the unit holding
// position X from the block counts of all sequences (lane l holds
// sequences 4l..4l+3, B <= 256); the work-group then walks, unit by unit,
// the blocks of [X, Y).  A whole unit's output is written here; a piece
// goes to record 2c (the share's first piece) or 2c + 1 (its last: a unit
// that starts in the share and runs past its end), and the piece that
// holds a unit's block 0 also records where the unit's pieces are for the
// merge.  The share of position z is the largest c' with c' T / S <= z,
// i.e. ((z + 1) S - 1) / T.
template <int PF, bool DBG, bool KV8>
__device__ __forceinline__ void even_walk(const DecodeArgs& a, int tab_tokens, int32_t* bt_s,
                                          float* merge_s) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int W = blockDim.x / kWave;
  const int G = a.G, Hkv = a.Hkv;
  const int K = a.even_kappa;
  int nb[4], cx[4], len[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = 4 * lane + i;
    const int raw = idx < a.B ? a.ctx[idx] : 0;
    cx[i] = raw < 0 ? 0 : (raw > tab_tokens ? tab_tokens : raw);
    nb[i] = (cx[i] + kT - 1) / kT;
    len[i] = nb[i] > 0 ? nb[i] + K : 0;
    if (DBG && raw > tab_tokens && a.dbg_err) atomicOr(a.dbg_err, 2);
  }
  const int mine = len[0] + len[1] + len[2] + len[3];
  const int incl = wave_prefix_i32(mine);
  const int N = __builtin_amdgcn_readlane(incl, kWave - 1);
  const int T = N * Hkv;
  const int S = gridDim.x;
  const int c = blockIdx.x;
  const int X = (int)((int64_t)c * T / S);
  const int Y = (int)((int64_t)(c + 1) * T / S);
  // no blocks: an empty record at 2c, for the merge of a unit that spans
  // this share (only a share with no positions can lie inside a unit's
  // span without blocks of it; any other share without blocks is read by
  // no merge, and gets the same record)
  auto empty_record = [&]() {
    for (int idx = tid; idx < G * kD; idx += blockDim.x) {
      const int h = idx / kD, d = idx % kD;
      const int64_t r = (int64_t)2 * c * G + h;
      a.ws_o[r * kD + d] = 0.f;
      if (d == 0) {
        a.ws_ml[r * 2] = -INFINITY;
        a.ws_ml[r * 2 + 1] = 0.f;
      }
    }
  };
  if (X == Y) {
    empty_record();
    return;
  }
  int kvh = X / N;
  const int xr = X - kvh * N;  // X's position among head kvh's
  int start = incl - mine;
  int fb = -1, frel = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (xr >= start && xr < start + len[i]) {
      fb = 4 * lane + i;
      frel = xr - start;
    }
    start += len[i];
  }
  const int ol = __builtin_ctzll(__builtin_amdgcn_ballot_w64(fb >= 0));
  int b = __builtin_amdgcn_readlane(fb, ol);
  int vs = X - __builtin_amdgcn_readlane(frel, ol);  // the unit's first position
  auto pick = [&](const int* v, int seq) {  // v[seq % 4] of the lane holding seq
    const int k = seq & 3;
    const int x = k == 0 ? v[0] : k == 1 ? v[1] : k == 2 ? v[2] : v[3];
    return __builtin_amdgcn_readlane(x, seq >> 2);
  };
  int nbb = pick(nb, b);
  int pos = X;
  bool first = true;
  // the next unit with blocks after (b, kvh), KV-head-major; kvh2 == Hkv if none
  auto next_unit = [&](int& b2, int& kvh2) {
    int n = 0;
    while (true) {
      if (++b2 >= a.B) {
        b2 = 0;
        if (++kvh2 >= Hkv) return 0;
      }
      n = pick(nb, b2);
      if (n > 0) return n;
    }
  };
  while (true) {
    // this unit's blocks inside [pos, Y)
    const int r0 = (pos > vs + K ? pos : vs + K) - (vs + K);
    const int r1 = (Y < vs + K + nbb ? Y : vs + K + nbb) - (vs + K);
    if (r1 > r0) {
      walk_range<PF, DBG, KV8>(a, b, kvh, pick(cx, b), r0, r1, bt_s, merge_s);
      const bool whole = r0 == 0 && r1 == nbb;
      const int rec = first ? 2 * c : 2 * c + 1;
      if (r0 == 0 && tid == 0) {
        const int64_t last = (int64_t)vs + K + nbb - 1;  // the unit's last block
        const int c1 = (int)(((last + 1) * S - 1) / T);
        a.ws_np[2 * (b * Hkv + kvh)] = rec;
        a.ws_np[2 * (b * Hkv + kvh) + 1] = c1 - c + 1;
      }
      for (int idx = tid; idx < G * kD; idx += blockDim.x) {
        const int h = idx / kD, d = idx % kD;
        float M, L, O;
        combine_waves(merge_s, W, G, h, d, M, L, O);
        if (whole) {
          a.out[((int64_t)b * a.Hq + kvh * G + h) * kD + d] =
              f32_to_f16_bits(O * a.v_scale / L);
        } else {
          const int64_t r = (int64_t)rec * G + h;
          a.ws_o[r * kD + d] = O;
          if (d == 0) {
            a.ws_ml[r * 2] = M;
            a.ws_ml[r * 2 + 1] = L;
          }
        }
      }
      first = false;
    }
    pos = vs + K + nbb;
    if (pos >= Y) break;
    // the next unit (one exists: pos < Y <= T); units are contiguous
    nbb = next_unit(b, kvh);
    if (kvh >= Hkv) break;  // not reached
    vs = pos;
    __syncthreads();  // the merge records above are read before the next walk
  }
  if (first) empty_record();  // no blocks in this share
}

// TWO selects the two-loop walk (fp16, no debug outputs), EVEN the even
// split (its own instances, so that its registers do not count against the
// other plans' occupancy).
template <int PF, bool DBG, bool KV8, bool TWO = false, bool EVEN = false>
__global__ void __launch_bounds__(512) pa_decode_kernel(const DecodeArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  int32_t* bt_s = reinterpret_cast<int32_t*>(smem_raw);
  float* merge_s = reinterpret_cast<float*>(smem_raw + a.lds_bt_bytes);

  // Debug timeline: the work-group's start and end on the constant 100 MHz
  // clock, and the HW_ID and XCC_ID registers of its CU (full 32 bits).
  int64_t* tl = nullptr;
  if constexpr (DBG) {
    if (a.dbg_timeline) {
      const int64_t wg =
          blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
      tl = a.dbg_timeline + wg * 4;
      if (threadIdx.x == 0) {
        tl[0] = (int64_t)__builtin_amdgcn_s_memrealtime();
        tl[2] = (int64_t)(uint32_t)__builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_ID
        tl[3] = (int64_t)(uint32_t)__builtin_amdgcn_s_getreg((31 << 11) | 20);  // XCC_ID
      }
    }
  }
  // every return below is taken by the whole work-group
  auto stamp_end = [&]() {
    if constexpr (DBG) {
      if (tl) {
        __syncthreads();
        if (threadIdx.x == 0) tl[1] = (int64_t)__builtin_amdgcn_s_memrealtime();
      }
    }
  };

  // Partition index slowest: every sequence's first partition is dispatched
  // before any second one, so the large work-groups of a ragged batch start
  // first and the short tail partitions fill in behind them.
  const int kvh = blockIdx.x;
  const int p = blockIdx.z;
  const int G = a.G;
  const int tid = threadIdx.x;
  const int W = blockDim.x / kWave;
  const int tab_tokens = a.MB * kT;
  if constexpr (EVEN) {
    even_walk<PF, DBG, KV8>(a, tab_tokens, bt_s, merge_s);
    stamp_end();
    return;
  }
  if (!a.balanced && a.chain == 2) {
    // Two sequences in turn, one partition each: grid row y takes ranks y
    // and B-1-y (B is even).
    for (int k = 0; k < 2; ++k) {
      if (k == 1) __syncthreads();  // the first sequence's merge records are read
      const int r = k == 0 ? (int)blockIdx.y : a.B - 1 - (int)blockIdx.y;
      const int bk = a.rank_seqs ? ranked_sequence(a, r, tab_tokens, smem_raw) : r;
      int ck = a.ctx[bk];
      if (ck > tab_tokens) {
        if (DBG && tid == 0 && a.dbg_err) atomicOr(a.dbg_err, 2);
        ck = tab_tokens;
      }
      const int nbk = ck > 0 ? (ck + kT - 1) / kT : 0;
      if (nbk == 0) {  // context <= 0: zeros
        for (int idx = tid; idx < G * kD; idx += blockDim.x) {
          const int h = idx / kD, d = idx % kD;
          a.out[((int64_t)bk * a.Hq + kvh * G + h) * kD + d] = 0;
        }
        continue;
      }
      if constexpr (!TWO) walk_range<PF, DBG, KV8>(a, bk, kvh, ck, 0, nbk, bt_s, merge_s);
      for (int idx = tid; idx < G * kD; idx += blockDim.x) {
        const int h = idx / kD, d = idx % kD;
        float M, L, O;
        combine_waves(merge_s, W, G, h, d, M, L, O);
        a.out[((int64_t)bk * a.Hq + kvh * G + h) * kD + d] =
            f32_to_f16_bits(O * a.v_scale / L);
      }
    }
    stamp_end();
    return;
  }
  int b, part = p, np_seq = a.P, pb = a.PB, ctx;
  if (a.balanced) {
    const Slot sl = balanced_slot(a, blockIdx.y, tab_tokens);
    if (sl.b < 0) {  // a grid row past the last partition
      stamp_end();
      return;
    }
    b = sl.b;
    part = sl.p;
    np_seq = sl.np;
    pb = sl.pb;
    ctx = sl.ctx;
    // the reduce takes each sequence's partition count from here
    if (part == 0 && kvh == 0 && tid == 0) a.ws_np[b] = np_seq;
  } else {
    b = a.rank_seqs ? ranked_sequence(a, blockIdx.y, tab_tokens, smem_raw) : blockIdx.y;
    ctx = a.ctx[b];
  }
  if (ctx > tab_tokens) {
    if (DBG && tid == 0 && a.dbg_err) atomicOr(a.dbg_err, 2);
    ctx = tab_tokens;
  }
  const int nb = ctx > 0 ? (ctx + kT - 1) / kT : 0;
  const int s = part * pb;
  const int e = min(nb, s + pb);

  if (s >= e) {
    // Nothing to attend in this partition.  With one partition the output
    // rows are written here (context <= 0 gives zeros); otherwise the reduce
    // kernel only reads partitions that hold blocks.
    if (a.P == 1) {
      for (int idx = tid; idx < G * kD; idx += blockDim.x) {
        const int h = idx / kD, d = idx % kD;
        a.out[((int64_t)b * a.Hq + kvh * G + h) * kD + d] = 0;
      }
    }
    stamp_end();
    return;
  }

  if constexpr (TWO) {
    float* logit_s = merge_s + W * G * kRec;
    walk_two_loop<PF>(a, b, kvh, ctx, s, e, bt_s, merge_s, logit_s, logit_s + a.PB * kT * G);
  } else {
    walk_range<PF, DBG, KV8>(a, b, kvh, ctx, s, e, bt_s, merge_s);
  }

  for (int idx = tid; idx < G * kD; idx += blockDim.x) {
    const int h = idx / kD, d = idx % kD;
    float M, L, O;
    combine_waves(merge_s, W, G, h, d, M, L, O);
    const int64_t row = (int64_t)b * a.Hq + kvh * G + h;
    if (a.P == 1 || np_seq == 1) {  // the sequence's only partition
      a.out[row * kD + d] = f32_to_f16_bits(O * a.v_scale / L);
    } else {
      const int64_t pr = row * a.P + part;
      if (d == 0) {
        a.ws_ml[pr * 2] = M;
        a.ws_ml[pr * 2 + 1] = L;
      }
      a.ws_o[pr * kD + d] = O;
    }
  }
  stamp_end();
}

// ---------------------------------------------------------------------------
// Cross-partition combine: one work-group of 128 threads per (sequence, head).
// Its time is latency.  The (m, l) pairs of the first kReduceRegs
// partitions (one cache line) and the outputs of the first `spec` of them
// are loaded together with the context length (and, under the balanced
// split, the sequence's partition count) before either is known, so one
// memory round trip precedes the arithmetic when the sequence has at most
// `spec` partitions.  spec is the plan's partition count, or under the
// balanced split the count every sequence of a uniform batch gets: loading
// further speculative outputs would read workspace lines that no partition
// wrote (straight from HBM).  Outputs between spec and the sequence's count
// are loaded once it is known.  Every branch combines in the same order, so
// the results are the same bits.
// Merge of the even split's pieces of one (sequence, head) row, in piece
// order.  The context length and the unit's record are loaded together;
// then the (m, l, o) of the first kReduceRegs pieces, together.  More
// pieces: the maximum first, then the sums, in chunks of kReduceRegs whose
// loads are issued together (the same order of operations).
__device__ __forceinline__ void reduce_even(const DecodeArgs& a) {
  const int row = blockIdx.x;  // b * Hq + h
  const int b = row / a.Hq, h = row % a.Hq;
  const int kvh = h / a.G, g = h % a.G;
  const int d = threadIdx.x;
  const int rec0 = a.ws_np[2 * (b * a.Hkv + kvh)];
  int np = a.ws_np[2 * (b * a.Hkv + kvh) + 1];
  int ctx = a.ctx[b];
  ctx = min(ctx, a.MB * kT);
  if (ctx <= 0) {
    a.out[(int64_t)row * kD + d] = 0;
    return;
  }
  if (rec0 < 0 || rec0 >= 2 * a.shares) {  // not written by the decode kernel: NaN
    a.out[(int64_t)row * kD + d] = 0x7E00;
    return;
  }
  if (np <= 1) return;  // the decode kernel wrote this row
  const int c0 = rec0 >> 1;
  np = np < a.shares - c0 ? np : a.shares - c0;  // the records stay inside the workspace
  auto rec = [&](int j) { return (int64_t)(j == 0 ? rec0 : 2 * (c0 + j)) * a.G + g; };
  float mq[kReduceRegs], lq[kReduceRegs], oq[kReduceRegs];
  auto load = [&](int j0) {
#pragma unroll
    for (int i = 0; i < kReduceRegs; ++i) {
      if (j0 + i < np) {
        const int64_t r = rec(j0 + i);
        mq[i] = a.ws_ml[r * 2];
        lq[i] = a.ws_ml[r * 2 + 1];
        oq[i] = a.ws_o[r * kD + d];
      }
    }
  };
  float M = -INFINITY;
  if (np <= kReduceRegs) {
    load(0);
#pragma unroll
    for (int i = 0; i < kReduceRegs; ++i)
      if (i < np) M = fmaxf(M, mq[i]);
  } else {
    for (int j0 = 0; j0 < np; j0 += kReduceRegs) {
#pragma unroll
      for (int i = 0; i < kReduceRegs; ++i)
        if (j0 + i < np) mq[i] = a.ws_ml[rec(j0 + i) * 2];
#pragma unroll
      for (int i = 0; i < kReduceRegs; ++i)
        if (j0 + i < np) M = fmaxf(M, mq[i]);
    }
  }
  float L = 0.f, O = 0.f;
  for (int j0 = 0; j0 < np; j0 += kReduceRegs) {
    if (np > kReduceRegs) load(j0);
#pragma unroll
    for (int i = 0; i < kReduceRegs; ++i) {
      if (j0 + i < np) {
        const float al = fast_exp2(mq[i] - M);
        L += al * lq[i];
        O += al * oq[i];
      }
    }
  }
  a.out[(int64_t)row * kD + d] = f32_to_f16_bits(O * a.v_scale / L);
}

__global__ void __launch_bounds__(128) pa_reduce_kernel(const DecodeArgs a) {
  if (a.even) {
    reduce_even(a);
    return;
  }
  const int row = blockIdx.x;  // b * Hq + h
  const int b = row / a.Hq;
  const int d = threadIdx.x;
  const float* ml = a.ws_ml + (int64_t)row * a.P * 2;
  const float* o = a.ws_o + (int64_t)row * a.P * kD;
  const int spec = a.balanced ? a.k_uniform : a.P;
  float mq[kReduceRegs], lq[kReduceRegs], oq[kReduceRegs];
#pragma unroll
  for (int q = 0; q < kReduceRegs; ++q) {
    if (q < a.P) {
      mq[q] = ml[2 * q];
      lq[q] = ml[2 * q + 1];
    }
    if (q < spec) oq[q] = o[(int64_t)q * kD + d];
  }
  int ctx = a.ctx[b];
  const int np_b = a.balanced ? a.ws_np[b] : 0;
  ctx = min(ctx, a.MB * kT);
  const int nb = ctx > 0 ? (ctx + kT - 1) / kT : 0;
  const int np = nb == 0 ? 0 : (a.balanced ? np_b : (nb + a.PB - 1) / a.PB);
  if (np == 0) {
    a.out[(int64_t)row * kD + d] = 0;
    return;
  }
  if (a.balanced && np == 1) return;  // the decode kernel wrote this row
  if (np <= kReduceRegs) {
#pragma unroll
    for (int q = 0; q < kReduceRegs; ++q)
      if (q >= spec && q < np) oq[q] = o[(int64_t)q * kD + d];
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < kReduceRegs; ++q)
      if (q < np) M = fmaxf(M, mq[q]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int q = 0; q < kReduceRegs; ++q) {
      if (q < np) {
        const float al = fast_exp2(mq[q] - M);
        L += al * lq[q];
        O += al * oq[q];
      }
    }
    a.out[(int64_t)row * kD + d] = f32_to_f16_bits(O * a.v_scale / L);
    return;
  }
  // more partials: the maximum first, then the sums in chunks of
  // kReduceRegs whose loads are issued together (same order of operations)
  float M = -INFINITY;
  for (int q = 0; q < np; ++q) M = fmaxf(M, ml[2 * q]);
  float L = 0.f, O = 0.f;
  for (int q0 = 0; q0 < np; q0 += kReduceRegs) {
#pragma unroll
    for (int i = 0; i < kReduceRegs; ++i) {
      if (q0 + i < np) {
        mq[i] = ml[2 * (q0 + i)];
        lq[i] = ml[2 * (q0 + i) + 1];
        oq[i] = o[(int64_t)(q0 + i) * kD + d];
      }
    }
#pragma unroll
    for (int i = 0; i < kReduceRegs; ++i) {
      if (q0 + i < np) {
        const float al = fast_exp2(mq[i] - M);
        L += al * lq[i];
        O += al * oq[i];
      }
    }
  }
  a.out[(int64_t)row * kD + d] = f32_to_f16_bits(O * a.v_scale / L);
}

// ---------------------------------------------------------------------------
// Streaming-read ceiling: every 16-byte word of buf read once.  Each wave
// reads whole 8 KiB chunks (8 non-temporal 128-bit loads per lane, 1 KiB
// contiguous per instruction, the decode kernel's access granularity), the
// chunks dealt round-robin over all waves; a ragged tail is read word by
// word.  One XOR per work-group goes to sink so no load is dead.
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* __restrict__ buf,
                                                          int64_t n16, u32x4* sink) {
  constexpr int kChunkWords = 512;  // 8 KiB
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave_id = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x / kWave);
  const int64_t nchunks = n16 / kChunkWords;
  u32x4 x = {0u, 0u, 0u, 0u};
  for (int64_t ch = wave_id; ch < nchunks; ch += nwaves) {
    const u32x4* p = buf + ch * kChunkWords + lane;
    u32x4 r[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = __builtin_nontemporal_load(p + kWave * k);
#pragma unroll
    for (int k = 0; k < 8; ++k) x ^= r[k];
  }
  const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = nchunks * kChunkWords + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
       i < n16; i += nthreads)
    x ^= __builtin_nontemporal_load(buf + i);
  // reduce within the work-group so only one value per group is stored
  __shared__ u32x4 red[256];
  red[threadIdx.x] = x;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if ((int)threadIdx.x < st) red[threadIdx.x] ^= red[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

// ---------------------------------------------------------------------------
// Launchers.

template <int PF, bool DBG, bool KV8, bool TWO = false, bool EVEN = false>
static hipError_t launch_decode_t(const DecodeArgs& a, dim3 grid, dim3 block, size_t lds,
                                  hipStream_t st) {
  hipLaunchKernelGGL((pa_decode_kernel<PF, DBG, KV8, TWO, EVEN>), grid, block, lds, st, a);
  return hipGetLastError();
}

template <int PF, bool DBG, bool KV8>
static hipError_t launch_even_t(const DecodeArgs& a, dim3 grid, dim3 block, size_t lds,
                                hipStream_t st) {
  return launch_decode_t<PF, DBG, KV8, false, true>(a, grid, block, lds, st);
}

hipError_t launch_decode(const DecodeArgs& a, int pf, bool dbg, bool kv8, int waves,
                         size_t lds, hipStream_t st) {
  typedef hipError_t (*fn_t)(const DecodeArgs&, dim3, dim3, size_t, hipStream_t);
  // pf 0..3 are the look-ahead modes; 4 is the register look-ahead of depth
  // 2, 5 and 6 the LDS ring of depth 1 and 2
  static const fn_t table[28] = {
      launch_decode_t<0, false, false>, launch_decode_t<0, true, false>,
      launch_decode_t<1, false, false>, launch_decode_t<1, true, false>,
      launch_decode_t<2, false, false>, launch_decode_t<2, true, false>,
      launch_decode_t<3, false, false>, launch_decode_t<3, true, false>,
      launch_decode_t<4, false, false>, launch_decode_t<4, true, false>,
      launch_decode_t<5, false, false>, launch_decode_t<5, true, false>,
      launch_decode_t<6, false, false>, launch_decode_t<6, true, false>,
      launch_decode_t<0, false, true>,  launch_decode_t<0, true, true>,
      launch_decode_t<1, false, true>,  launch_decode_t<1, true, true>,
      launch_decode_t<2, false, true>,  launch_decode_t<2, true, true>,
      launch_decode_t<3, false, true>,  launch_decode_t<3, true, true>,
      launch_decode_t<4, false, true>,  launch_decode_t<4, true, true>,
      launch_decode_t<5, false, true>,  launch_decode_t<5, true, true>,
      launch_decode_t<6, false, true>,  launch_decode_t<6, true, true>};
  static const fn_t even_table[28] = {
      launch_even_t<0, false, false>, launch_even_t<0, true, false>,
      launch_even_t<1, false, false>, launch_even_t<1, true, false>,
      launch_even_t<2, false, false>, launch_even_t<2, true, false>,
      launch_even_t<3, false, false>, launch_even_t<3, true, false>,
      launch_even_t<4, false, false>, launch_even_t<4, true, false>,
      launch_even_t<5, false, false>, launch_even_t<5, true, false>,
      launch_even_t<6, false, false>, launch_even_t<6, true, false>,
      launch_even_t<0, false, true>,  launch_even_t<0, true, true>,
      launch_even_t<1, false, true>,  launch_even_t<1, true, true>,
      launch_even_t<2, false, true>,  launch_even_t<2, true, true>,
      launch_even_t<3, false, true>,  launch_even_t<3, true, true>,
      launch_even_t<4, false, true>,  launch_even_t<4, true, true>,
      launch_even_t<5, false, true>,  launch_even_t<5, true, true>,
      launch_even_t<6, false, true>,  launch_even_t<6, true, true>};
  if (pf < 0 || pf > 6) return hipErrorInvalidValue;
  const dim3 grid = a.even ? dim3(a.shares)
                           : dim3(a.Hkv, a.balanced ? a.nslot : a.B / a.chain,
                                  a.balanced ? 1 : a.P);
  const dim3 block(kWave * waves);
  // what the walk needs (the LDS ring: depth + 1 slots of one block's K and
  // V per wave); the plan may ask for more, to cap the residency
  const size_t slots = pf >= 5 ? (size_t)waves * (pf - 3) * (kv8 ? 4096 : 8192) : 0;
  const size_t need =
      decode_lds_bytes(a.balanced ? a.pb_max : a.PB, a.G, waves, a.B, a.rank_seqs != 0, slots);
  const int k = (kv8 ? 14 : 0) + pf * 2 + (dbg ? 1 : 0);
  return (a.even ? even_table : table)[k](a, grid, block, lds > need ? lds : need, st);
}

hipError_t launch_decode_two_loop(const DecodeArgs& a, int pf, int waves, size_t lds,
                                  hipStream_t st) {
  typedef hipError_t (*fn_t)(const DecodeArgs&, dim3, dim3, size_t, hipStream_t);
  static const fn_t table[4] = {
      launch_decode_t<0, false, false, true>, launch_decode_t<1, false, false, true>,
      launch_decode_t<2, false, false, true>, launch_decode_t<3, false, false, true>};
  if (pf < 0 || pf > 3) return hipErrorInvalidValue;
  const dim3 grid(a.Hkv, a.B, a.P);
  const dim3 block(kWave * waves);
  const size_t need = two_loop_lds_bytes(a.PB, a.G, waves, a.B, a.rank_seqs != 0);
  return table[pf](a, grid, block, lds > need ? lds : need, st);
}

hipError_t launch_reduce(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(pa_reduce_kernel, dim3((unsigned)(a.B * a.Hq)), dim3(kD), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// K from the token-major layout to the grouped one.  A (block, head) slice is
// 16 token rows of R 16-byte pieces (R = 16 for fp16, 8 for E4M3); piece
// (t, g) of the input becomes piece (g, t) of the output.  Each thread moves
// one piece per step of a grid-stride loop, so every load instruction reads
// 1 KiB of contiguous input.
__global__ void __launch_bounds__(256) pack_k_kernel(const u32x4* __restrict__ in,
                                                     u32x4* __restrict__ out, int64_t slices,
                                                     int R) {
  const int64_t per = 16 * (int64_t)R;  // pieces per slice
  const int64_t total = slices * per;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t sl = i / per;
    const int p = (int)(i - sl * per);
    const int t = p / R, g = p - t * R;
    out[sl * per + g * 16 + t] = in[i];
  }
}

// ---------------------------------------------------------------------------
// Scratch of the no-allocation entry point: the partition partials of calls
// that cannot allocate.  Every GPU the library runs on holds its own copy
// for the life of the process.  On the host, `noalloc_scratch_array` names a
// host-side stand-in, never a device address: its device address is looked
// up once per device (with that device current) and cached.
static __device__ __align__(256) unsigned char noalloc_scratch_array[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch_array));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_pack_k(const void* in, void* out, int64_t slices, bool kv8, hipStream_t st) {
  const int R = kv8 ? 8 : 16;
  const int64_t pieces = slices * 16 * R;
  int64_t groups = (pieces + 255) / 256;
  if (groups > 65536) groups = 65536;  // grid-stride beyond
  hipLaunchKernelGGL(pack_k_kernel, dim3((unsigned)groups), dim3(256), 0, st,
                     reinterpret_cast<const u32x4*>(in), reinterpret_cast<u32x4*>(out), slices, R);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, size_t bytes, void* sink, int groups,
                              hipStream_t st) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(groups), dim3(256), 0, st,
                     reinterpret_cast<const u32x4*>(buf), (int64_t)(bytes / 16),
                     reinterpret_cast<u32x4*>(sink));
  return hipGetLastError();
}

}  // namespace pa
